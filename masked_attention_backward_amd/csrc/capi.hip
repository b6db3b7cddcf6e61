// C ABI of the masked attention library: host-side validation of scalars and pointer
// values, workspace carving, and kernel enqueueing on the caller's stream.
//
// The host does shapes, offsets and launches only (page "knowledge(triton) ... #174",
// BlockSparseAttentionGrad runbook, "optimisation 1": the host only checks shapes,
// allocates and views).  Nothing here reads device memory, allocates, or synchronises.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "maskattn.h"
#include "ma_launch.h"

using ma::AttnArgs;

namespace {

constexpr int kMaxDim = 65535;    // grid y/z limits of the preprocess launch

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per-row fp32 buffers (Delta, lse * log2 e) are padded to a multiple of 64 rows per head.
size_t pad64(int S) { return ((size_t)S + 63) & ~(size_t)63; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool tensor_ok(const void* p) { return p != nullptr && aligned(p, 16); }

// Rows of one [B, H, S] tensor must stay well inside int32 grid/row arithmetic.
bool sizes_fit(long long B, long long H, long long S) {
  return B * H * S <= (1ll << 31) - 1 && B * H * ((S + 63) / 64) <= (1ll << 31) - 1;
}

int check_common(int B, int Hq, int Hkv, int S, int D, float scale, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || D < 1) return MA_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return MA_EINVAL;
  if (Hq % Hkv != 0) return MA_EINVAL;
  if (D != ma::HD) return MA_EUNSUPPORTED;
  if (dtype != MA_F16 && dtype != MA_BF16) return MA_EUNSUPPORTED;
  if (B > kMaxDim || Hq > kMaxDim) return MA_EUNSUPPORTED;
  if (!sizes_fit(B, Hq, S)) return MA_EUNSUPPORTED;
  return MA_OK;
}

int check_blocks(int bx, int by) {
  if (bx < 1 || by < 1) return MA_EINVAL;
  if (bx % 16 != 0 || by % 16 != 0 || bx > 128 || by > 128) return MA_EUNSUPPORTED;
  return MA_OK;
}

// Block path: a dK/dV workgroup walks at most this many selected query blocks (summed over the
// query heads of its group); key blocks selected more often are split over several
// workgroups whose fp32 partial sums a reduce kernel adds in a fixed order.
constexpr int kBlockChunk = 32;

// Chunks per (kv head, key block) the dK/dV grid provides: ceil(group * nqb / kBlockChunk),
// or 1 when a key block has at most 2 kBlockChunk possible entries (one workgroup then walks at
// most twice the usual count, which costs less than the partial sums, the reduce kernel and the
// idle chunk slots of a split that most shapes of this size never use).
int block_max_chunks(int N, int Nkv, int nqb) {
  const long long g = N / Nkv;
  if (g * nqb <= 2 * kBlockChunk) return 1;
  return (int)((g * nqb + kBlockChunk - 1) / kBlockChunk);
}

struct BlockLayout {
  size_t delta, lse2, mask_t, sel_q, cnt_q, sel_k, cnt_k, part, total;
};

// The partial-sum region is sized for any Nkv dividing N: Nkv * ceil((N / Nkv) * nqb / C) <=
// floor(N * (nqb + C - 1) / C) chunk slots per batch, each of padded Skv rows of D fp32 values,
// for dK and for dV.  It is absent when no key block can be split (N * nqb <= 2 kBlockChunk).
BlockLayout block_layout(int B, int N, int Sq, int Skv, int nqb, int nkb) {
  BlockLayout l;
  const size_t bn = (size_t)B * N;
  l.delta = 0;
  l.lse2 = align256(l.delta + bn * pad64(Sq) * sizeof(float));
  l.mask_t = align256(l.lse2 + bn * pad64(Sq) * sizeof(float));
  l.sel_q = align256(l.mask_t + bn * nkb * nqb);
  l.cnt_q = align256(l.sel_q + bn * nqb * nkb * sizeof(int32_t));
  l.sel_k = align256(l.cnt_q + bn * nqb * sizeof(int32_t));
  l.cnt_k = align256(l.sel_k + bn * nkb * nqb * sizeof(int32_t));
  l.part = align256(l.cnt_k + bn * nkb * sizeof(int32_t));
  l.total = l.part;
  if ((long long)N * nqb > 2 * kBlockChunk) {
    const size_t slots = (size_t)B * (((size_t)N * (nqb + kBlockChunk - 1)) / kBlockChunk);
    l.total = align256(l.part + 2 * slots * pad64(Skv) * ma::HD * sizeof(float));
  }
  return l;
}

AttnArgs base_args(const void* q, const void* k, const void* v, int B, int Hq, int Hkv, int Sq, int Skv,
                   float scale) {
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.group = Hq / Hkv;
  a.max_chunks = 1;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return a;
}

template <class T>
T* at(void* base, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

int status_of(hipError_t e) { return e == hipSuccess ? MA_OK : MA_ELAUNCH; }

}  // namespace

// Scratch memory of attn_sink_bwd_noalloc (Delta, lse * log2 e and the dsink partials, laid
// out as the attn_sink_bwd workspace): a file-scope device array, one copy per GPU, resident
// from the first use of the library on that GPU until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it only names the symbol): the device
// address is looked up once per device with hipGetSymbolAddress and kept below.
static __device__ __align__(256) unsigned char scratch[MA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call per device,
// with that device current).
hipError_t scratch_address(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = r;
    g_scratch_ptr[dev] = (r == hipSuccess) ? p : nullptr;
  });
  *out = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace

extern "C" {

const char* maskattn_strerror(int status) {
  switch (status) {
    case MA_OK: return "ok";
    case MA_EINVAL: return "invalid argument (null or misaligned pointer, bad size, Hq % Hkv != 0, window < 1)";
    case MA_EUNSUPPORTED: return "unsupported configuration (D != 128, block size, dtype or size limits)";
    case MA_EWORKSPACE: return "workspace too small";
    case MA_ELAUNCH: return "HIP runtime error while enqueueing";
    case MA_ESCRATCH:
      return "problem needs more scratch than attn_sink_bwd_noalloc's static array holds "
             "(MA_NOALLOC_SCRATCH_BYTES); use attn_sink_bwd with a workspace";
    default: return "unknown status";
  }
}

int attn_sink_fwd(const void* q, const void* k, const void* v, const float* sink, void* o, float* lse, int B,
                  int Hq, int Hkv, int S, int D, int window, float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, S, D, scale, dtype);
  if (st) return st;
  if (window < 1) return MA_EINVAL;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return MA_EINVAL;
  if (!sink || !aligned(sink, 4) || !lse || !aligned(lse, 4)) return MA_EINVAL;
  AttnArgs a = base_args(q, k, v, B, Hq, Hkv, S, S, scale);
  a.sink = sink;
  a.out_o = o;
  a.out_lse = lse;
  a.window = window < S ? window : S;
  return status_of(ma::launch_fwd(dtype, a, ma::MASK_WINDOW, (hipStream_t)stream));
}

size_t attn_sink_bwd_workspace_bytes(int B, int Hq, int Hkv, int S, int D) {
  if (check_common(B, Hq, Hkv, S, D, 1.f, MA_F16) != MA_OK) return 0;
  const size_t rows = align256((size_t)B * Hq * pad64(S) * sizeof(float));
  const size_t nblk = (size_t)B * Hq * ((S + 63) / 64);
  return align256(2 * rows + nblk * sizeof(float));
}

// dS bank of the window path: live 32 x 32 blocks per (sequence, query head), kb below the
// diagonal for window W (clamped to S), 2048 bytes per block.
static long long ds_kb_of(int S, int window) {
  const int W = window < S ? window : S;
  return (W - 1 + 31) / 32;
}
static long long ds_blocks_of(int S, int window) { return ma::band_offset((S + 31) / 32, ds_kb_of(S, window)); }

// Head split of the dK/dV work on dense sequences whose key tiles give too few workgroups to
// fill the GPU: wide windows (128-row key tiles) with fewer than 256 tile pairs, where one
// workgroup per key tile would leave the heaviest tile (the first, under a causal window) with
// about twice the average work; narrow windows (64-row key tiles, two workgroups per compute
// unit) with fewer than 512 key tiles, whose few workgroups each walk a long chain of tiles
// whose copies cannot be hidden.  Each tile's visits (query heads x 64-row query tiles) are
// split over at most `group` workgroups of whole heads, at most a quarter of a compute unit's
// share of all visits each (at least one visit; a half and an eighth measured no faster on
// B1 H64 Hkv8 S4096); their fp32 partial sums are added in a fixed order.  max_chunks = 1: no
// split.
struct WindowSplit {
  int target, max_chunks;
};
static WindowSplit window_split(int B, int Hq, int Hkv, int S, int window) {
  WindowSplit ws{0, 1};
  const int W = window < S ? window : S;
  const int bc = ma::window_key_rows(W);
  const int nt = (S + bc - 1) / bc;
  const long long units = (long long)B * Hkv;
  if (ma::window_wide(W) ? units * ((nt + 1) / 2) >= 256 : units * nt >= 512) return ws;
  const int group = Hq / Hkv;
  long long visits = 0;
  for (int p = 0; p < nt; ++p) visits += (long long)group * ma::window_qtiles(S, W, p);
  const long long t = (units * visits + 1023) / 1024;
  ws.target = (int)(t < 1 ? 1 : t > (1ll << 30) ? (1ll << 30) : t);
  for (int p = 0; p < nt; ++p) {
    const int c = ma::window_chunks(S, W, group, ws.target, p);
    if (c > ws.max_chunks) ws.max_chunks = c;
  }
  return ws;
}
// The split's partial sums: dK and dV, max_chunks slots of padded S rows x D fp32 per
// (sequence, kv head).
static size_t window_part_bytes(int B, int Hkv, int S, const WindowSplit& ws) {
  if (ws.max_chunks <= 1) return 0;
  return align256(2 * (size_t)B * Hkv * ws.max_chunks * pad64(S) * ma::HD * sizeof(float));
}

size_t attn_sink_bwd_ds_workspace_bytes(int B, int Hq, int Hkv, int S, int D, int window) {
  const size_t base = attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D);
  if (base == 0 || window < 1) return 0;
  return base + align256((size_t)B * Hq * (size_t)ds_blocks_of(S, window) * 2048) +
         window_part_bytes(B, Hkv, S, window_split(B, Hq, Hkv, S, window));
}

static int sink_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, const float* sink, void* dq, void* dk, void* dv, float* dsink,
                         void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int window,
                         float scale, int dtype, void* stream, void* const* events, const int* cu = nullptr,
                         int total = 0) {
  int st = check_common(B, Hq, Hkv, S, D, scale, dtype);
  if (st) return st;
  if (window < 1) return MA_EINVAL;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dout) || !tensor_ok(dq) ||
      !tensor_ok(dk) || !tensor_ok(dv))
    return MA_EINVAL;
  if (!lse || !aligned(lse, 4) || !sink || !aligned(sink, 4) || !dsink || !aligned(dsink, 4)) return MA_EINVAL;
  if (!workspace || !aligned(workspace, 256)) return MA_EINVAL;
  const size_t need = attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D);
  if (workspace_bytes < need) return MA_EWORKSPACE;
  hipStream_t hs = (hipStream_t)stream;
  const size_t rows = align256((size_t)B * Hq * pad64(S) * sizeof(float));
  float* delta = at<float>(workspace, 0);
  float* lse2 = at<float>(workspace, rows);
  float* part = at<float>(workspace, 2 * rows);

  if (events) hipEventRecord((hipEvent_t)events[0], hs);
  hipError_t e = ma::launch_preprocess(dtype, o, dout, lse, sink, delta, lse2, part, B, Hq, S, hs, cu, total);
  if (e != hipSuccess) return MA_ELAUNCH;
  if (events) hipEventRecord((hipEvent_t)events[1], hs);
  AttnArgs a = base_args(q, k, v, B, Hq, Hkv, S, S, scale);
  // dsink from the preprocess's partials, by the first dK/dV workgroup (no launch of its own).
  a.dsink_part = part;
  a.dsink_out = dsink;
  a.dsink_nblk = (S + 63) / 64;
  a.dout = dout;
  a.lse = lse;
  a.lse2 = lse2;
  a.delta = delta;
  a.sink = sink;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu = cu;
  a.total = total;
  a.window = window < S ? window : S;
  // A workspace large enough for the dS bank selects the dQ path that reads the dS blocks the
  // dK/dV kernel stores (one GEMM per block) instead of recomputing S and dP.
  if (workspace_bytes >= attn_sink_bwd_ds_workspace_bytes(B, Hq, Hkv, S, D, window) &&
      ds_blocks_of(S, window) < (1ll << 30)) {
    a.ds_bank = at<uint16_t>(workspace, need);
    a.ds_kb = (int)ds_kb_of(S, window);
    a.ds_blocks = ds_blocks_of(S, window);
    // The same workspace holds the head split's partial sums after the bank (dense sequences).
    const WindowSplit ws = window_split(B, Hq, Hkv, S, window);
    if (!cu && ws.max_chunks > 1) {
      a.chunk = ws.target;
      a.max_chunks = ws.max_chunks;
      a.dkv_part = at<float>(workspace, need + align256((size_t)B * Hq * (size_t)ds_blocks_of(S, window) * 2048));
    }
  }
  e = ma::launch_window_bwd(dtype, a, hs, events ? (hipEvent_t)events[2] : nullptr);
  if (events) hipEventRecord((hipEvent_t)events[3], hs);
  return status_of(e);
}

int attn_sink_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  const float* sink, void* dq, void* dk, void* dv, float* dsink, void* workspace,
                  size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int window, float scale, int dtype,
                  void* stream) {
  return sink_bwd_impl(q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, workspace, workspace_bytes, B, Hq, Hkv, S, D,
                       window, scale, dtype, stream, nullptr);
}

int attn_sink_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const float* sink, void* dq, void* dk, void* dv, float* dsink,
                        void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int S, int D, int window,
                        float scale, int dtype, void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3]) return MA_EINVAL;
  return sink_bwd_impl(q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, workspace, workspace_bytes, B, Hq, Hkv, S, D,
                       window, scale, dtype, stream, events);
}

int attn_sink_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, const float* sink, void* dq, void* dk, void* dv, float* dsink, int B,
                          int Hq, int Hkv, int S, int D, int window, float scale, int dtype, void* stream) {
  const int st = check_common(B, Hq, Hkv, S, D, scale, dtype);
  if (st) return st;
  if (window < 1) return MA_EINVAL;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o) || !tensor_ok(dout) || !tensor_ok(dq) ||
      !tensor_ok(dk) || !tensor_ok(dv))
    return MA_EINVAL;
  if (!lse || !aligned(lse, 4) || !sink || !aligned(sink, 4) || !dsink || !aligned(dsink, 4)) return MA_EINVAL;
  const size_t need = attn_sink_bwd_workspace_bytes(B, Hq, Hkv, S, D);
  if (need > (size_t)MA_NOALLOC_SCRATCH_BYTES) return MA_ESCRATCH;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess || ws == nullptr) return MA_ELAUNCH;
  // Exactly the minimum workspace: the recompute dQ path, whatever the array could hold.
  return sink_bwd_impl(q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, ws, need, B, Hq, Hkv, S, D, window, scale,
                       dtype, stream, nullptr);
}

// Packed sequences: B sequences of at most max_seqlen rows at offsets cu_seqlens[0..B] of
// [H, total, D] tensors; scalar checks only (the offsets are device data).
static int varlen_check(const int* cu_seqlens, int B, int total, int max_seqlen, int Hq) {
  if (!cu_seqlens || !aligned(cu_seqlens, 4)) return MA_EINVAL;
  if (total < 1 || max_seqlen < 1 || max_seqlen > total) return MA_EINVAL;
  if (!sizes_fit(1, Hq, total)) return MA_EUNSUPPORTED;
  return MA_OK;
}

int attn_sink_fwd_varlen(const void* q, const void* k, const void* v, const float* sink, const int* cu_seqlens,
                         void* o, float* lse, int B, int total, int max_seqlen, int Hq, int Hkv, int D, int window,
                         float scale, int dtype, void* stream) {
  int st = check_common(B, Hq, Hkv, max_seqlen, D, scale, dtype);
  if (st) return st;
  st = varlen_check(cu_seqlens, B, total, max_seqlen, Hq);
  if (st) return st;
  if (window < 1) return MA_EINVAL;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(o)) return MA_EINVAL;
  if (!sink || !aligned(sink, 4) || !lse || !aligned(lse, 4)) return MA_EINVAL;
  AttnArgs a = base_args(q, k, v, B, Hq, Hkv, max_seqlen, max_seqlen, scale);
  a.sink = sink;
  a.out_o = o;
  a.out_lse = lse;
  a.cu = cu_seqlens;
  a.total = total;
  a.window = window < max_seqlen ? window : max_seqlen;
  return status_of(ma::launch_fwd(dtype, a, ma::MASK_WINDOW, (hipStream_t)stream));
}

int attn_sink_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, const float* sink, const int* cu_seqlens, void* dq, void* dk, void* dv,
                         float* dsink, void* workspace, size_t workspace_bytes, int B, int total, int max_seqlen,
                         int Hq, int Hkv, int D, int window, float scale, int dtype, void* stream) {
  const int st = varlen_check(cu_seqlens, B, total, max_seqlen, Hq);
  if (st) return st;
  return sink_bwd_impl(q, k, v, o, dout, lse, sink, dq, dk, dv, dsink, workspace, workspace_bytes, B, Hq, Hkv,
                       max_seqlen, D, window, scale, dtype, stream, nullptr, cu_seqlens, total);
}

int blocksparse_build_tables(const uint8_t* block_mask, int B, int N, int nqb, int nkb, uint8_t* mask_t,
                             int32_t* sel_q, int32_t* cnt_q, int32_t* sel_k, int32_t* cnt_k, void* stream) {
  if (B < 1 || N < 1 || nqb < 1 || nkb < 1) return MA_EINVAL;
  if (B > kMaxDim || N > kMaxDim || (long long)B * N > (1ll << 31) - 1) return MA_EUNSUPPORTED;
  if ((long long)nqb * nkb > (1ll << 30)) return MA_EUNSUPPORTED;
  if (!block_mask || !mask_t || !sel_q || !cnt_q || !sel_k || !cnt_k) return MA_EINVAL;
  if (!aligned(sel_q, 4) || !aligned(cnt_q, 4) || !aligned(sel_k, 4) || !aligned(cnt_k, 4)) return MA_EINVAL;
  return status_of(ma::launch_mask_tables(block_mask, B * N, nqb, nkb, mask_t, sel_q, cnt_q, sel_k, cnt_k,
                                          (hipStream_t)stream));
}

size_t blocksparse_attn_bwd_workspace_bytes(int B, int N, int Sq, int Skv, int D, int bx, int by) {
  if (check_common(B, N, N, Sq, D, 1.f, MA_F16) != MA_OK || Skv < 1 || check_blocks(bx, by) != MA_OK) return 0;
  if (!sizes_fit(B, N, Skv)) return 0;
  const int nqb = (Sq + bx - 1) / bx, nkb = (Skv + by - 1) / by;
  return block_layout(B, N, Sq, Skv, nqb, nkb).total;
}

// dS bank of the block path: one 2048-byte entry per (query head, 32-row query half, key
// sub-block) of a dense grid, key sub-block kb ceil(by/32) + j holding key rows kb by + 32 j ..
// of mask block kb (when by is a multiple of 32 that is the global 32-row key block, and the
// grid has ceil(Skv/32) of them; otherwise nkb ceil(by/32)); only entries inside selected
// mask blocks are written and read.  Kept below 2^30 entries per head (32-bit offsets in the
// kernels).
static long long block_bank_nka(int Skv, int by) {
  return by % 32 == 0 ? (Skv + 31) / 32 : (long long)((Skv + by - 1) / by) * ((by + 31) / 32);
}
static bool block_bank_ok(int Sq, int Skv, int bx, int by) {
  return bx % 16 == 0 && by % 16 == 0 && (long long)((Sq + 31) / 32) * block_bank_nka(Skv, by) < (1ll << 30);
}

size_t blocksparse_attn_bwd_ds_workspace_bytes(int B, int N, int Sq, int Skv, int D, int bx, int by) {
  const size_t base = blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, D, bx, by);
  if (base == 0 || !block_bank_ok(Sq, Skv, bx, by)) return base;
  return base + align256((size_t)B * N * (size_t)((Sq + 31) / 32) * (size_t)block_bank_nka(Skv, by) * 2048);
}

static int block_common(const void* q, const void* k, const void* v, const uint8_t* block_mask, void* workspace,
                        size_t workspace_bytes, int B, int N, int Nkv, int Sq, int Skv, int D, int bx, int by,
                        float scale, int dtype) {
  int st = check_common(B, N, Nkv, Sq, D, scale, dtype);
  if (st) return st;
  if (Skv < 1) return MA_EINVAL;
  if (!sizes_fit(B, N, Skv) || !sizes_fit(B, Nkv, Skv)) return MA_EUNSUPPORTED;
  st = check_blocks(bx, by);
  if (st) return st;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !block_mask) return MA_EINVAL;
  if (!workspace || !aligned(workspace, 256)) return MA_EINVAL;
  if (workspace_bytes < blocksparse_attn_bwd_workspace_bytes(B, N, Sq, Skv, D, bx, by)) return MA_EWORKSPACE;
  const int nqb = (Sq + bx - 1) / bx, nkb = (Skv + by - 1) / by;
  if ((long long)B * Nkv * nkb * block_max_chunks(N, Nkv, nqb) > 0x7fffffffll) return MA_EUNSUPPORTED;
  return MA_OK;
}

int blocksparse_attn_fwd_gqa(const void* q, const void* k, const void* v, const uint8_t* block_mask, void* o,
                             float* lse, void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Sq,
                             int Skv, int D, int bx, int by, float scale, int dtype, void* stream) {
  const int N = Hq;
  int st = block_common(q, k, v, block_mask, workspace, workspace_bytes, B, Hq, Hkv, Sq, Skv, D, bx, by, scale,
                        dtype);
  if (st) return st;
  if (!tensor_ok(o) || !lse || !aligned(lse, 4)) return MA_EINVAL;
  const int nqb = (Sq + bx - 1) / bx, nkb = (Skv + by - 1) / by;
  const BlockLayout L = block_layout(B, N, Sq, Skv, nqb, nkb);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = ma::launch_mask_tables(block_mask, B * N, nqb, nkb, at<uint8_t>(workspace, L.mask_t),
                                        at<int>(workspace, L.sel_q), at<int>(workspace, L.cnt_q),
                                        at<int>(workspace, L.sel_k), at<int>(workspace, L.cnt_k), hs);
  if (e != hipSuccess) return MA_ELAUNCH;
  AttnArgs a = base_args(q, k, v, B, Hq, Hkv, Sq, Skv, scale);
  a.out_o = o;
  a.out_lse = lse;
  a.mask = block_mask;
  a.sel_q = at<int>(workspace, L.sel_q);
  a.cnt_q = at<int>(workspace, L.cnt_q);
  a.sel_k = at<int>(workspace, L.sel_k);
  a.cnt_k = at<int>(workspace, L.cnt_k);
  a.bx = bx;
  a.by = by;
  a.nqb = nqb;
  a.nkb = nkb;
  return status_of(ma::launch_fwd(dtype, a, ma::MASK_BLOCK, hs));
}

int blocksparse_attn_fwd(const void* q, const void* k, const void* v, const uint8_t* block_mask, void* o, float* lse,
                         void* workspace, size_t workspace_bytes, int B, int N, int Sq, int Skv, int D, int bx,
                         int by, float scale, int dtype, void* stream) {
  return blocksparse_attn_fwd_gqa(q, k, v, block_mask, o, lse, workspace, workspace_bytes, B, N, N, Sq, Skv, D, bx,
                                  by, scale, dtype, stream);
}

static int block_bwd_impl(const void* q, const void* k, const void* v, const void* o, const void* dout,
                          const float* lse, const uint8_t* block_mask, void* dq, void* dk, void* dv,
                          void* workspace, size_t workspace_bytes, int B, int N, int Nkv, int Sq, int Skv, int D,
                          int bx, int by, float scale, int dtype, void* stream, void* const* events) {
  int st = block_common(q, k, v, block_mask, workspace, workspace_bytes, B, N, Nkv, Sq, Skv, D, bx, by, scale,
                        dtype);
  if (st) return st;
  if (!tensor_ok(o) || !tensor_ok(dout) || !tensor_ok(dq) || !tensor_ok(dk) || !tensor_ok(dv)) return MA_EINVAL;
  if (!lse || !aligned(lse, 4)) return MA_EINVAL;
  const int nqb = (Sq + bx - 1) / bx, nkb = (Skv + by - 1) / by;
  const BlockLayout L = block_layout(B, N, Sq, Skv, nqb, nkb);
  hipStream_t hs = (hipStream_t)stream;
  if (events) hipEventRecord((hipEvent_t)events[0], hs);
  float* delta = at<float>(workspace, L.delta);
  float* lse2 = at<float>(workspace, L.lse2);
  hipError_t e = ma::launch_block_prep(dtype, block_mask, B, N, nqb, nkb, at<uint8_t>(workspace, L.mask_t),
                                       at<int>(workspace, L.sel_q), at<int>(workspace, L.cnt_q),
                                       at<int>(workspace, L.sel_k), at<int>(workspace, L.cnt_k), o, dout, lse,
                                       delta, lse2, Sq, hs);
  if (e != hipSuccess) return MA_ELAUNCH;
  if (events) hipEventRecord((hipEvent_t)events[1], hs);
  AttnArgs a = base_args(q, k, v, B, N, Nkv, Sq, Skv, scale);
  a.dout = dout;
  a.lse = lse;
  a.lse2 = lse2;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.mask = block_mask;
  a.sel_q = at<int>(workspace, L.sel_q);
  a.cnt_q = at<int>(workspace, L.cnt_q);
  a.sel_k = at<int>(workspace, L.sel_k);
  a.cnt_k = at<int>(workspace, L.cnt_k);
  a.bx = bx;
  a.by = by;
  a.nqb = nqb;
  a.nkb = nkb;
  a.max_chunks = block_max_chunks(N, Nkv, nqb);
  if (a.max_chunks > 1) {
    a.chunk = kBlockChunk;
    a.dkv_part = at<float>(workspace, L.part);
  } else {
    a.max_chunks = 1;
  }
  // A workspace large enough for the dS bank selects the dQ path that reads the dS blocks the
  // dK/dV kernel stores instead of recomputing S and dP.
  if (block_bank_ok(Sq, Skv, bx, by) &&
      workspace_bytes >= blocksparse_attn_bwd_ds_workspace_bytes(B, N, Sq, Skv, D, bx, by)) {
    a.ds_bank = at<uint16_t>(workspace, L.total);
    a.ds_nka = (int)block_bank_nka(Skv, by);
    a.ds_blocks = (long long)((Sq + 31) / 32) * a.ds_nka;
  }
  e = ma::launch_block_bwd(dtype, a, hs, events ? (hipEvent_t)events[2] : nullptr);
  if (events) hipEventRecord((hipEvent_t)events[3], hs);
  return status_of(e);
}

int blocksparse_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, const uint8_t* block_mask, void* dq, void* dk, void* dv, void* workspace,
                         size_t workspace_bytes, int B, int N, int Sq, int Skv, int D, int bx, int by, float scale,
                         int dtype, void* stream) {
  return block_bwd_impl(q, k, v, o, dout, lse, block_mask, dq, dk, dv, workspace, workspace_bytes, B, N, N, Sq, Skv,
                        D, bx, by, scale, dtype, stream, nullptr);
}

int blocksparse_attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const void* dout,
                             const float* lse, const uint8_t* block_mask, void* dq, void* dk, void* dv, void* workspace,
                             size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Skv, int D, int bx, int by,
                             float scale, int dtype, void* stream) {
  return block_bwd_impl(q, k, v, o, dout, lse, block_mask, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Sq,
                        Skv, D, bx, by, scale, dtype, stream, nullptr);
}

int blocksparse_attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dout,
                               const float* lse, const uint8_t* block_mask, void* dq, void* dk, void* dv,
                               void* workspace, size_t workspace_bytes, int B, int N, int Sq, int Skv, int D, int bx,
                               int by, float scale, int dtype, void* stream, void* const* events) {
  if (!events || !events[0] || !events[1] || !events[2] || !events[3]) return MA_EINVAL;
  return block_bwd_impl(q, k, v, o, dout, lse, block_mask, dq, dk, dv, workspace, workspace_bytes, B, N, N, Sq, Skv,
                        D, bx, by, scale, dtype, stream, events);
}

}  // extern "C"
