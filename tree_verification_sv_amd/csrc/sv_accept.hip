// Speculative acceptance and the bonus token.
//
// "Accelerating Sonar Through Speculation" (Perplexity), sections
// "Decodificacion Especulativa" and "EAGLE": the longest acceptable draft
// sequence is kept and the target logits after it yield one extra token, so
// n drafted tokens emit up to n+1; section "Objetivo-Borrador": acceptance
// compares the full draft and target distributions; section "Inferencia con
// Decodificacion Especulativa": the accepted count stays on the device here,
// so no host sync is needed.  "Speculative Speculative Decoding", sec. 3B:
// after a rejection the residual mass max(0, p - q) carries the next draw.
//
// Row decomposition.  At row r (distributions p = p_r, q = q_r) the children
// are tested in ascending index.  After k rejections the current distribution
// is max(0, p - c_k q) / S(c_k), with S(c) = sum_v max(0, p(v) - c q(v)),
// c_0 = 0, S(c_0) = 1 and c_k = c_{k-1} + S(c_{k-1}): one rejection maps
// max(0, p - c q)/S(c) to max(0, p - (c + S(c)) q)/S(c + S(c)).  The walk only
// stops at a row after every child was rejected, so both the first accepted
// child of a row and the bonus token drawn if the walk stops there depend on
// that row alone.  Every row is therefore resolved independently and in
// parallel, and the walk is a pointer chase over the per-row results.
//
// Work decomposition.  A group of G work-groups resolves one row; each of TH
// threads (512 greedy; 256, or 512 in large batches, for the walk modes) owns a
// slice of TH * 128 bytes of the vocabulary (greedy batches of 512 rows or
// more: G = 1, and the work-group streams the whole row slice by slice with the
// next slice's loads in flight).  Thread t owns the 16-byte pieces k * TH + t
// (k = 0 .. 7) of its slice, so every load instruction of a wave reads 1 KB of
// consecutive logits.
// The exponentials are computed once into registers; each later pass over the row (a
// rejection's residual sum, the bonus scan) is a few register operations per
// entry.  Members of a group trade per-slice partials through tagged 64-bit
// words (tag and payload in one atomic word, so a reader that sees the tag
// also sees the value).  Greedy rows need one pass (slice max / argmax, lowest
// id on ties).  Rows resolved: the root row and the rows with a usable child
// (a walk that stops at a row without one needs only that row's argmax or its
// target distribution, which the walker's work-group takes itself); stochastic
// chains and narrow trees also resolve the rows of all other usable nodes (leaf
// rows read the target logits only).  The work-groups of other rows exit at
// once.
//
// The walk.  Greedy, and stochastic chains or narrow trees (N <= 2 max_depth,
// where nearly every row is on the path): the group that completes the last
// row of a sequence walks.  Stochastic wide trees: the walk advances as rows
// resolve -- a per-sequence frontier names the first row of the accepted path
// not resolved yet; the work-group that publishes that row takes the frontier
// over and follows the path through the rows already resolved, until it either
// reaches the stop row (it writes the outputs and raises the sequence's cancel
// flag, so its other rows stop at their next exchange) or hands the frontier
// to the next unresolved row.  Off-path rows then cost nothing after the walk.
//
// Forward progress.  Work-groups are dispatched in index order, round-robin
// over the 8 XCDs; the members of a group are consecutive in their XCD's
// dispatch order (block indices x, x + 8, ..., x + 8 (G - 1)), and a member
// only ever waits for members of its own group.  Every group ahead of the
// oldest unfinished one has finished, so that group is resident or next in
// line: no group waits for a work-group that cannot start.  The waits are
// bounded all the same (status SV_SEQ_TIMEOUT).
#include <mutex>

#include "sv_accept_dev.h"

namespace {

// PRE: fetch the target slice before the sequence facts (stochastic chains and narrow trees,
// which resolve nearly every row); without it, wide trees resolve only the rows with a usable
// child and the walker draws a stop row without children itself
template <typename T, int MODE, bool ALIGNED, int TH, bool PRE>
__global__ void __launch_bounds__(TH, 2) k_accept(sv_accept_args a, int32_t G, AccWs ws,
                                                                  sv_commit_args cm, int32_t has_cm) {
  constexpr bool STO = MODE != SV_GREEDY;
  __shared__ AccShared<T, TH, STO> S;
  const AccRole role{(int)blockIdx.x, (int)gridDim.x, (a.N + 1) * G};
  accept_body<T, MODE, ALIGNED, TH, PRE>(a, G, ws, cm, has_cm, role, S);
}

// greedy batches of at least AC_STREAM_ROWS rows and fewer than AC_CHAIN_B sequences: the
// needed rows as one list.  bf16 rows on 16 bytes fit two work-groups per CU (four waves per
// SIMD, 128 registers) without spilling; the other forms keep one work-group per CU.
template <typename T, bool ALIGNED>
constexpr int rows_wgs_per_cu() { return ALIGNED && sizeof(T) == 2 ? 2 : 1; }
template <typename T, bool ALIGNED>
__global__ void __launch_bounds__(512, (2 * rows_wgs_per_cu<T, ALIGNED>()))
    k_accept_rows(sv_accept_args a, AccWs ws, sv_commit_args cm, int32_t has_cm) {
  __shared__ AccShared<T, 512, false> S;
  greedy_rows_body<T, ALIGNED, 512, false>(a, 0, ws, cm, has_cm, S);
}
// ... and of AC_CHAIN_B sequences or more: a chain per sequence, G work-groups per row
// (THR: threshold acceptance, mode 3)
template <typename T, bool ALIGNED, bool THR = false>
__global__ void __launch_bounds__(AC_CHAIN_TH, 2)
    k_accept_chain(sv_accept_args a, int32_t G, AccWs ws, sv_commit_args cm, int32_t has_cm) {
  __shared__ AccShared<T, AC_CHAIN_TH, false> S;
  greedy_rows_body<T, ALIGNED, AC_CHAIN_TH, true, THR>(a, G, ws, cm, has_cm, S);
}

// SV_FLAG_VALIDATE: one work-group per logits row (target rows, then draft rows in mode 1) looks
// for a NaN or +Inf entry, or a row without any finite entry, and sets status 8 for the
// sequence unless the acceptance already reported a code.
template <typename T>
__device__ __forceinline__ void nf_check(T x, bool& bad, bool& finite);
template <>
__device__ __forceinline__ void nf_check<uint16_t>(uint16_t h, bool& bad, bool& finite) {
  const bool fin = (h & 0x7f80u) != 0x7f80u;
  finite |= fin;
  bad |= !fin && h != 0xff80u;  // NaN or +Inf (-Inf is probability 0)
}
template <>
__device__ __forceinline__ void nf_check<float>(float x, bool& bad, bool& finite) {
  const bool fin = isfinite(x);
  finite |= fin;
  bad |= !fin && !(x < 0.f && isinf(x));
}
template <typename T>
__global__ void __launch_bounds__(256) k_nonfinite_rows(const T* __restrict__ target, const T* __restrict__ draft,
                                                        int32_t B, int32_t R, int32_t V, int32_t* __restrict__ status) {
  __shared__ int s_any_bad, s_any_fin;
  const int64_t row = blockIdx.x;  // [0, B*R) target rows, [B*R, 2*B*R) draft rows
  const int64_t nrows = (int64_t)B * R;
  const T* p = (row < nrows ? target + row * V : draft + (row - nrows) * V);
  const int b = (int)((row < nrows ? row : row - nrows) / R);
  if (threadIdx.x == 0) { s_any_bad = 0; s_any_fin = 0; }
  __syncthreads();
  bool bad = false, fin = false;
  for (int v = threadIdx.x; v < V; v += 256) nf_check<T>(p[v], bad, fin);
  if (bad) s_any_bad = 1;
  if (fin) s_any_fin = 1;
  __syncthreads();
  if (threadIdx.x == 0 && (s_any_bad || !s_any_fin)) atomicCAS(&status[b], 0, SV_SEQ_NONFINITE);
}

template <typename T, int M, bool AL>
void launch_accept(int TH, dim3 grid, hipStream_t st, const sv_accept_args& a, int G, const AccWs& ws,
                   const sv_commit_args& cm, int32_t has_cm) {
  // the walk modes prefetch unless the walk advances as rows resolve (wide trees: only rows with a
  // usable child are resolved, and 512-thread groups are only taken for wide trees); fp32 logits
  // (the small-vocabulary path) always prefetch and resolve every row, which keeps those kernels
  // free of the walker's leaf draw and of its register pressure
  constexpr bool LEAF = sizeof(T) == 2;
  const bool pre = !LEAF || !(a.N > 2 * a.max_depth);
  if constexpr (M == SV_GREEDY) {
    if (G == 1) {  // rows read whole: a chain per sequence, or the batch's needed rows as one list
      if (rows_chain(a)) {
        const int CG = chain_G(a);
        hipLaunchKernelGGL((k_accept_chain<T, AL>), dim3((unsigned)chain_grid(a, CG)), dim3(AC_CHAIN_TH), 0, st, a, CG, ws,
                           cm, has_cm);
      } else {
        hipLaunchKernelGGL((k_accept_rows<T, AL>), dim3((unsigned)rows_grid(a, rows_wgs_per_cu<T, AL>())), dim3(512), 0, st,
                           a, ws, cm, has_cm);
      }
    } else {
      hipLaunchKernelGGL((k_accept<T, M, AL, 512, true>), grid, dim3(512), 0, st, a, G, ws, cm, has_cm);
    }
  } else if constexpr (AL) {
    if (TH == 512) hipLaunchKernelGGL((k_accept<T, M, AL, 512, !LEAF>), grid, dim3(512), 0, st, a, G, ws, cm, has_cm);
    else if (pre) hipLaunchKernelGGL((k_accept<T, M, AL, 256, true>), grid, dim3(256), 0, st, a, G, ws, cm, has_cm);
    else if constexpr (LEAF) hipLaunchKernelGGL((k_accept<T, M, AL, 256, false>), grid, dim3(256), 0, st, a, G, ws, cm, has_cm);
  } else {  // rows off 16 bytes: always 256 threads (acc_threads)
    if (pre) hipLaunchKernelGGL((k_accept<T, M, AL, 256, true>), grid, dim3(256), 0, st, a, G, ws, cm, has_cm);
    else if constexpr (LEAF) hipLaunchKernelGGL((k_accept<T, M, AL, 256, false>), grid, dim3(256), 0, st, a, G, ws, cm, has_cm);
  }
}

// SV_FLAG_VALIDATE, after the acceptance kernels: scan every logits row the call could read,
// then wait and read the status back.
sv_status validate_logits(const sv_accept_args& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.B * (a.N + 1) * (a.mode == SV_STOCHASTIC ? 2 : 1);
  if (rows > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  if (a.logits_dtype == SV_BF16)
    hipLaunchKernelGGL(k_nonfinite_rows<uint16_t>, dim3((unsigned)rows), dim3(256), 0, st,
                       (const uint16_t*)a.target_logits, (const uint16_t*)a.draft_logits, a.B, a.N + 1, a.V, a.status);
  else
    hipLaunchKernelGGL(k_nonfinite_rows<float>, dim3((unsigned)rows), dim3(256), 0, st,
                       (const float*)a.target_logits, (const float*)a.draft_logits, a.B, a.N + 1, a.V, a.status);
  const sv_status ls = sv_launch_status();
  if (ls != SV_OK) return ls;
  return sv_validate_status(a.status, a.B, st);
}

}  // namespace

extern "C" size_t sv_accept_workspace(const sv_accept_args* args) {
  if (!args || args->B < 1 || args->N < 1 || args->V < 1) return 0;
  if (args->mode == SV_THRESHOLD) {  // either form (chains or row statistics): the larger
    const size_t c = ws_layout(*args).total, r = sv_threshold_workspace(*args);
    return c > r ? c : r;
  }
  return ws_layout(*args).total;
}

extern "C" sv_status sv_accept(const sv_accept_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  const sv_accept_args& a = *args;
  if (a.B < 0 || a.N < 1 || a.N > SV_MAX_N || a.V < 1 || a.max_depth < 1 || a.max_depth > SV_MAX_DEPTH)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.mode != SV_GREEDY && a.mode != SV_STOCHASTIC && a.mode != SV_TOPK_DRAFT && a.mode != SV_THRESHOLD)
    return SV_ERR_INVALID_ARGUMENT;
  if (a.logits_dtype != SV_F32 && a.logits_dtype != SV_BF16) return SV_ERR_UNSUPPORTED;
  if (a.mode == SV_THRESHOLD && (!(a.temperature > 0.f) || !(a.threshold >= 0.f && a.threshold <= 1.f)))
    return SV_ERR_INVALID_ARGUMENT;
  if (a.flags & ~(uint32_t)(SV_FLAG_VALIDATE | SV_FLAG_ROW_LIST)) return SV_ERR_INVALID_ARGUMENT;
  if (a.B == 0) return SV_OK;
  // modes 0, 1 and 2 read neither mask output when depth is NULL (depths come from the parents)
  const bool mask_free = a.mode != SV_THRESHOLD && !a.depth;
  if (!a.parents || !a.tokens || (!mask_free && (!a.anc_bits || !a.depth)) || !a.target_logits || !a.accept_len || !a.accept_rows ||
      !a.out_tokens || !a.num_out || !a.stop_row || !a.status || !a.workspace)
    return SV_ERR_INVALID_ARGUMENT;
  sv_commit_args cm{};
  if (a.commit) {  // the walker commits the accepted path itself
    const sv_status cs = svc::walker_commit_ok(*a.commit, a.B, a.N, a.max_depth);
    if (cs != SV_OK) return cs;
    cm = *a.commit;
  }
  const int32_t has_cm = a.commit != nullptr;
  const bool validate = (a.flags & SV_FLAG_VALIDATE) != 0;
  if (validate) {
    if (a.mode == SV_STOCHASTIC && !a.draft_logits) return SV_ERR_INVALID_ARGUMENT;
    const sv_status r = sv_validate_ready((hipStream_t)stream);
    if (r != SV_OK) return r;
  }
  if (a.mode == SV_THRESHOLD) {
    if ((uintptr_t)a.workspace % 256) return SV_ERR_INVALID_ARGUMENT;
    sv_status r;
    // chains along the passing paths (k_accept_chain, mode 3) for rows on 16 bytes
    const size_t esz = a.logits_dtype == SV_BF16 ? 2 : 4;
    const bool al = ((size_t)a.V * esz) % 16 == 0 && ((uintptr_t)a.target_logits % 16) == 0;
    if (al && thr_chain(a)) {
      const WsLayout l = ws_layout(a);
      if (a.workspace_bytes < l.total) return SV_ERR_INVALID_ARGUMENT;
      const AccWs ws = ws_views(a.workspace, l);
      const int CG = chain_G(a);
      const dim3 grid((unsigned)chain_grid(a, CG)), block(AC_CHAIN_TH);
      hipStream_t st = (hipStream_t)stream;
      if (a.logits_dtype == SV_BF16)
        hipLaunchKernelGGL((k_accept_chain<uint16_t, true, true>), grid, block, 0, st, a, CG, ws, cm, has_cm);
      else
        hipLaunchKernelGGL((k_accept_chain<float, true, true>), grid, block, 0, st, a, CG, ws, cm, has_cm);
      r = sv_launch_status();
    } else {
      r = sv_threshold_launch(a, cm, has_cm, (hipStream_t)stream);
    }
    if (r != SV_OK || !validate) return r;
    return validate_logits(a, (hipStream_t)stream);
  }
  if (a.mode == SV_STOCHASTIC && !a.draft_logits) return SV_ERR_INVALID_ARGUMENT;
  if (a.mode != SV_GREEDY && (!a.u_accept || !a.u_sample || !(a.temperature > 0.f))) return SV_ERR_INVALID_ARGUMENT;
  const WsLayout l = ws_layout(a);
  if (a.workspace_bytes < l.total || ((uintptr_t)a.workspace % 256)) return SV_ERR_INVALID_ARGUMENT;
  // rows start on 16 bytes when the row pitch and the base pointers are multiples of 16
  const size_t esz = a.logits_dtype == SV_BF16 ? 2 : 4;
  const bool aligned = ((size_t)a.V * esz) % 16 == 0 && ((uintptr_t)a.target_logits % 16) == 0 &&
                       (a.mode != SV_STOCHASTIC || ((uintptr_t)a.draft_logits % 16) == 0);
  const int TH = acc_threads(a, aligned);
  const int G = launch_G(a, TH);
  if (G > AC_MAXG) return SV_ERR_UNSUPPORTED;
  const int64_t blocks = num_groups(a) * G;
  if (blocks > 0x7fffffff) return SV_ERR_UNSUPPORTED;
  const AccWs ws = ws_views(a.workspace, l);
  hipStream_t st = (hipStream_t)stream;
  const dim3 grid((unsigned)blocks);
#define SV_ACC_LAUNCH(T, M, AL) launch_accept<T, M, AL>(TH, grid, st, a, G, ws, cm, has_cm)
  if (a.logits_dtype == SV_BF16) {
    if (a.mode == SV_STOCHASTIC) { if (aligned) SV_ACC_LAUNCH(uint16_t, SV_STOCHASTIC, true); else SV_ACC_LAUNCH(uint16_t, SV_STOCHASTIC, false); }
    else if (a.mode == SV_TOPK_DRAFT) { if (aligned) SV_ACC_LAUNCH(uint16_t, SV_TOPK_DRAFT, true); else SV_ACC_LAUNCH(uint16_t, SV_TOPK_DRAFT, false); }
    else { if (aligned) SV_ACC_LAUNCH(uint16_t, SV_GREEDY, true); else SV_ACC_LAUNCH(uint16_t, SV_GREEDY, false); }
  } else {
    if (a.mode == SV_STOCHASTIC) { if (aligned) SV_ACC_LAUNCH(float, SV_STOCHASTIC, true); else SV_ACC_LAUNCH(float, SV_STOCHASTIC, false); }
    else if (a.mode == SV_TOPK_DRAFT) { if (aligned) SV_ACC_LAUNCH(float, SV_TOPK_DRAFT, true); else SV_ACC_LAUNCH(float, SV_TOPK_DRAFT, false); }
    else { if (aligned) SV_ACC_LAUNCH(float, SV_GREEDY, true); else SV_ACC_LAUNCH(float, SV_GREEDY, false); }
  }
#undef SV_ACC_LAUNCH
  const sv_status ls = sv_launch_status();
  if (ls != SV_OK || !validate) return ls;
  return validate_logits(a, st);
}

// ---------------------------------------------------------------- no-allocation variant
// sv_accept_noalloc runs sv_accept with a workspace that lives in the library itself: a
// file-scope device array of SV_ACCEPT_SCRATCH_BYTES, one copy per GPU, held until the
// process ends.  Its device address comes from hipGetSymbolAddress, taken once per device
// with that device current; host code never passes the array's own name to a kernel (on the
// host that name is a stand-in, not a device address).  The array starts zeroed (static
// storage) and is cleared once more by a fill kernel on the caller's stream the first time a
// device is used (a kernel, not a memset, so that the first call may sit inside a captured
// graph); every acceptance launch leaves the workspace zeroed again, as the workspace
// contract of sv_accept requires.  Every call on one GPU shares the array: calls that
// overlap in time on one GPU race.
static __device__ __align__(256) unsigned char scratch[SV_ACCEPT_SCRATCH_BYTES];

namespace {
constexpr int SV_SCRATCH_MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[SV_SCRATCH_MAX_DEVICES];

__global__ void __launch_bounds__(256) k_zero16(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The scratch array's device address on the current device (set up on first use).
sv_status scratch_for_current_device(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SV_ERR_HIP;
  if (dev < 0 || dev >= SV_SCRATCH_MAX_DEVICES) return SV_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SV_ERR_HIP;
    hipLaunchKernelGGL(k_zero16, dim3(256), dim3(256), 0, st, (uint4*)p, (size_t)SV_ACCEPT_SCRATCH_BYTES / 16);
    if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SV_OK;
}
}  // namespace

extern "C" sv_status sv_accept_noalloc(const sv_accept_args* args, void* stream) {
  if (!args) return SV_ERR_INVALID_ARGUMENT;
  sv_accept_args a = *args;
  a.workspace = nullptr;
  a.workspace_bytes = 0;
  if (a.B == 0) return sv_accept(&a, stream);  // argument checks only; nothing to launch
  const size_t need = sv_accept_workspace(&a);
  if (need == 0) return SV_ERR_INVALID_ARGUMENT;  // shape rejected by the workspace query
  if (need > (size_t)SV_ACCEPT_SCRATCH_BYTES) return SV_ERR_SCRATCH_LIMIT;
  void* p = nullptr;
  const sv_status s = scratch_for_current_device((hipStream_t)stream, &p);
  if (s != SV_OK) return s;
  a.workspace = p;
  a.workspace_bytes = (size_t)SV_ACCEPT_SCRATCH_BYTES;
  return sv_accept(&a, stream);
}
