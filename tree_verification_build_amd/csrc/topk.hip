// ddtree_draft_topk: per-depth top-K tokens of the draft head and their
// full-vocabulary log-probs.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's
// Tree-Parallel Evaluation Strategy", Section 1 step 1: every depth position
// of the draft's output gives top-k candidate tokens with log-probs, the
// input of the best-first tree build (step 2).  Readings: log-softmax of the
// row at temperature 1 over the whole vocabulary; candidates ordered by logit
// descending, ties to the lower token id.
//
// A row is streamed in S slices of 256 threads x EPT elements, each thread
// holding its elements in registers (coalesced loads: element e of thread t
// is slice start + 256 e + t).  Per slice:
//   * the slice maximum m and sum of exp(x - m) (the log-sum-exp partial);
//   * the top-K by packed key (order-preserving value bits << 32 | ~id, so a
//     larger key is a larger value or, for equal values, a lower id).  Every
//     wave finds the K-th largest of its 64 lane maxima; tau = the largest of
//     those four values.  At least K elements are >= tau (one wave's K lane
//     maxima), so the slice's top K are all among the candidates x >= tau,
//     which for real rows are a handful: when there are at most 64 of them,
//     wave 0 ranks them (one candidate per lane, ranks by comparing against
//     every other), otherwise (heavy ties) K rounds of a block-wide maximum
//     below the previous key pick them from the registers directly.
// A one-wave-per-row kernel merges the S slices' K keys (K rounds of a wave
// maximum below the previous key) and their (m, sum) pairs, and writes the
// tokens and log-probs x - lse.  With S = 1 the slice kernel writes them.
#include <algorithm>

#include "common.hpp"

namespace ddt {
namespace {

constexpr int kTkThreads = 256;
constexpr int kTkWaves = kTkThreads / kWave;
constexpr int kTkMaxCand = 64;

template <typename T> __device__ __forceinline__ float tk_get(const T* p, long i);
template <> __device__ __forceinline__ float tk_get<float>(const float* p, long i) { return p[i]; }
template <> __device__ __forceinline__ float tk_get<uint16_t>(const uint16_t* p, long i) {
  return bf16_to_f32(p[i]);
}

__device__ __forceinline__ uint64_t tk_key(float v, int idx) {
  return (static_cast<uint64_t>(ord_f32(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

// wave-uniform maximum through the order-preserving bits (DPP row maxima)
__device__ __forceinline__ float wave_max_f32(float v) { return unord_f32(wave_max_u32(ord_f32(v))); }

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += shfl_xor_f32(v, o);
  return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// K-th largest of the wave's 64 values, counting repeats (K <= 64).
__device__ __forceinline__ float wave_kth_largest(float v, int K, int lane) {
  float t = v;
  float kth = -__builtin_huge_valf();
  for (int j = 0; j < K; ++j) {
    kth = wave_max_f32(t);
    const uint64_t at = __ballot(t == kth);
    if (at == 0) break;   // only when every value is NaN-free -inf already taken
    if (lane == __builtin_ctzll(at)) t = -__builtin_huge_valf();
  }
  return kth;
}

__device__ __forceinline__ void write_result(uint64_t key, float lse, int32_t* tok, float* lp) {
  if (key == 0) {            // fewer than K elements in the row
    *tok = -1;
    *lp = -__builtin_huge_valf();
    return;
  }
  *tok = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
  *lp = unord_f32(static_cast<uint32_t>(key >> 32)) - lse;
}

// Slices of one row: grid (S, rows).  Writes K keys (0 = none) and the
// (max, sum exp) pair of the slice, or the final outputs when S == 1.
template <typename T, int EPT>
__global__ __launch_bounds__(kTkThreads) void topk_slice_kernel(
    const T* __restrict__ logits, int V, int K, int S, int chunk, uint64_t* __restrict__ ws_key,
    float2* __restrict__ ws_ms, int32_t* __restrict__ tok, float* __restrict__ lp) {
  __shared__ float s_f[kTkWaves];
  __shared__ int s_i[kTkWaves];
  __shared__ uint64_t s_k[kTkWaves];
  __shared__ uint64_t s_cand[kTkMaxCand];
  __shared__ uint64_t s_top[DDTREE_MAX_TOPK];
  const int sl = blockIdx.x, row = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const long start = static_cast<long>(sl) * chunk;
  const long end = min(static_cast<long>(V), start + chunk);
  const T* rp = logits + static_cast<long>(row) * V;

  float v[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const long i = start + static_cast<long>(e) * kTkThreads + tid;
    v[e] = i < end ? tk_get<T>(rp, i) : -__builtin_huge_valf();
  }
  float tmax = -__builtin_huge_valf();
#pragma unroll
  for (int e = 0; e < EPT; ++e) tmax = max(tmax, v[e]);

  // slice maximum, then the sum of exp(x - m)
  const float wm = wave_max_f32(tmax);
  // this wave's K-th largest lane maximum (independent of the block maximum)
  const float wk = wave_kth_largest(tmax, K, lane);
  if (lane == 0) {
    s_f[wave] = wm;
    s_k[wave] = __float_as_uint(wk);
  }
  __syncthreads();
  float m = s_f[0], tau = __uint_as_float(static_cast<uint32_t>(s_k[0]));
#pragma unroll
  for (int w = 1; w < kTkWaves; ++w) {
    m = max(m, s_f[w]);
    tau = max(tau, __uint_as_float(static_cast<uint32_t>(s_k[w])));
  }
  float se = 0.0f;
  int cnt = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    se += __expf(v[e] - m);
    const long i = start + static_cast<long>(e) * kTkThreads + tid;
    cnt += (i < end && v[e] >= tau) ? 1 : 0;
  }
  se = wave_sum_f32(se);
  const int wc = wave_sum_i32(cnt);
  __syncthreads();   // s_f / s_i reused below
  if (lane == 0) {
    s_f[wave] = se;
    s_i[wave] = wc;
  }
  __syncthreads();
  float ssum = 0.0f;
  int C = 0, wbase = 0;
#pragma unroll
  for (int w = 0; w < kTkWaves; ++w) {
    ssum += s_f[w];
    if (w < wave) wbase += s_i[w];
    C += s_i[w];
  }
  const float lse = m + __logf(ssum);   // used when S == 1

  if (C <= kTkMaxCand) {
    // compact the candidates into LDS: this thread's offset in its wave
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int o = __shfl_up(incl, d, kWave);
      if (lane >= d) incl += o;
    }
    int pos = wbase + incl - cnt;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const long i = start + static_cast<long>(e) * kTkThreads + tid;
      if (i < end && v[e] >= tau) s_cand[pos++] = tk_key(v[e], static_cast<int>(i));
    }
    __syncthreads();
    if (wave == 0) {
      const uint64_t mine = lane < C ? s_cand[lane] : 0ull;
      int rank = 0;
      for (int j = 0; j < C; ++j) {
        const uint64_t other = s_cand[j];
        rank += other > mine ? 1 : 0;
      }
      if (lane < C && rank < K) s_top[rank] = mine;
      if (lane >= C && lane < K) s_top[lane] = 0ull;   // fewer than K elements
    }
  } else {
    // heavy ties: K rounds of the block maximum below the previous key
    uint64_t prev = ~0ull;
    for (int j = 0; j < K; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const long i = start + static_cast<long>(e) * kTkThreads + tid;
        const uint64_t k = i < end ? tk_key(v[e], static_cast<int>(i)) : 0ull;
        best = (k < prev && k > best) ? k : best;
      }
      best = wave_max_u64(best);
      __syncthreads();
      if (lane == 0) s_k[wave] = best;
      __syncthreads();
      uint64_t b = s_k[0];
#pragma unroll
      for (int w = 1; w < kTkWaves; ++w) b = max(b, s_k[w]);
      if (tid == 0) s_top[j] = b;
      prev = b;
    }
  }
  __syncthreads();
  if (tid < K) {
    const uint64_t key = s_top[tid];
    if (S == 1) {
      write_result(key, lse, tok + static_cast<long>(row) * K + tid, lp + static_cast<long>(row) * K + tid);
    } else {
      ws_key[(static_cast<long>(row) * S + sl) * K + tid] = key;
    }
  }
  if (S > 1 && tid == 0) ws_ms[static_cast<long>(row) * S + sl] = make_float2(m, ssum);
}

// One wave per row: merge the S slices' keys and (max, sum) pairs.  With
// kLds the row's S*K keys and S pairs are first copied into LDS with all their
// loads in flight at once, so the K selection rounds and the two passes over
// the pairs cost one round trip to memory instead of one each.
constexpr int kMergeLdsBytes = 48 * 1024;

template <bool kLds>
__global__ __launch_bounds__(kWave) void topk_merge_kernel(int K, int S,
                                                            const uint64_t* __restrict__ ws_key,
                                                            const float2* __restrict__ ws_ms,
                                                            int32_t* __restrict__ tok,
                                                            float* __restrict__ lp) {
  __shared__ uint64_t s_top[DDTREE_MAX_TOPK];
  extern __shared__ uint64_t s_dyn[];   // kLds: S*K keys, then S pairs
  const int row = blockIdx.x, lane = threadIdx.x;
  const int n = S * K;
  const uint64_t* keys = ws_key + static_cast<long>(row) * n;
  const float2* ms = ws_ms + static_cast<long>(row) * S;
  if (kLds) {
    float2* s_ms = reinterpret_cast<float2*>(s_dyn + n);
    for (int i = lane; i < n; i += kWave) s_dyn[i] = keys[i];
    for (int i = lane; i < S; i += kWave) s_ms[i] = ms[i];
    __syncthreads();
    keys = s_dyn;
    ms = s_ms;
  }
  float m = -__builtin_huge_valf();
  for (int s = lane; s < S; s += kWave) m = max(m, ms[s].x);
  m = wave_max_f32(m);
  float sum = 0.0f;
  for (int s = lane; s < S; s += kWave) {
    const float2 p = ms[s];
    sum += p.y * __expf(p.x - m);
  }
  sum = wave_sum_f32(sum);
  const float lse = m + __logf(sum);
  uint64_t prev = ~0ull;
  for (int j = 0; j < K; ++j) {
    uint64_t best = 0;
    for (int i = lane; i < n; i += kWave) {
      const uint64_t k = keys[i];
      best = (k < prev && k > best) ? k : best;
    }
    best = wave_max_u64(best);
    if (lane == 0) s_top[j] = best;
    prev = best;
  }
  __syncthreads();
  if (lane < K)
    write_result(s_top[lane], lse, tok + static_cast<long>(row) * K + lane,
                 lp + static_cast<long>(row) * K + lane);
}

// Elements per thread and slice count: about 1024 workgroups over all rows,
// 4 to 32 elements per thread.
void topk_plan(int rows, int V, int* ept, int* S, int* chunk) {
  const long total = static_cast<long>(rows) * V;
  const long per = (total + 1024L * kTkThreads - 1) / (1024L * kTkThreads);
  int e = 4;
  while (e < 32 && e < per) e *= 2;
  *ept = e;
  *chunk = kTkThreads * e;
  *S = static_cast<int>((static_cast<long>(V) + *chunk - 1) / *chunk);
}

template <typename T, int EPT>
void launch_slices(const void* logits, int rows, int V, int K, int S, int chunk, uint64_t* wk,
                   float2* wm, int32_t* tok, float* lp, hipStream_t st) {
  hipLaunchKernelGGL((topk_slice_kernel<T, EPT>), dim3(S, rows), dim3(kTkThreads), 0, st,
                     static_cast<const T*>(logits), V, K, S, chunk, wk, wm, tok, lp);
}

template <typename T>
void launch_topk(int ept, const void* logits, int rows, int V, int K, int S, int chunk,
                 uint64_t* wk, float2* wm, int32_t* tok, float* lp, hipStream_t st) {
  switch (ept) {
    case 4: launch_slices<T, 4>(logits, rows, V, K, S, chunk, wk, wm, tok, lp, st); break;
    case 8: launch_slices<T, 8>(logits, rows, V, K, S, chunk, wk, wm, tok, lp, st); break;
    case 16: launch_slices<T, 16>(logits, rows, V, K, S, chunk, wk, wm, tok, lp, st); break;
    default: launch_slices<T, 32>(logits, rows, V, K, S, chunk, wk, wm, tok, lp, st); break;
  }
  if (S > 1) {
    const size_t lds = static_cast<size_t>(S) * (K + 1) * sizeof(uint64_t);
    if (lds <= kMergeLdsBytes)
      hipLaunchKernelGGL((topk_merge_kernel<true>), dim3(rows), dim3(kWave), lds, st, K, S, wk, wm,
                         tok, lp);
    else
      hipLaunchKernelGGL((topk_merge_kernel<false>), dim3(rows), dim3(kWave), 0, st, K, S, wk, wm,
                         tok, lp);
  }
}

size_t topk_ws_bytes(int rows, int S, int K) {
  if (S <= 1) return 0;
  return static_cast<size_t>(rows) * S * (static_cast<size_t>(K) * sizeof(uint64_t) + sizeof(float2));
}

}  // namespace
}  // namespace ddt

extern "C" size_t ddtree_draft_topk_workspace_size(int32_t rows, int32_t V, int32_t K) {
  if (rows < 1 || V < 1 || K < 1 || K > DDTREE_MAX_TOPK) return 0;
  int ept, S, chunk;
  ddt::topk_plan(rows, V, &ept, &S, &chunk);
  return ddt::topk_ws_bytes(rows, S, K);
}

extern "C" ddtree_status ddtree_draft_topk(const void* logits, ddtree_dtype dtype, int32_t rows,
                                           int32_t V, int32_t K, int32_t* tokens, float* logprobs,
                                           void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  using namespace ddt;
  if (!logits || !tokens || !logprobs) return fail(DDTREE_EINVAL, "ddtree_draft_topk: null pointer");
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "ddtree_draft_topk: unknown dtype %d", static_cast<int>(dtype));
  if (rows < 1 || V < 1)
    return fail(DDTREE_EINVAL, "ddtree_draft_topk: sizes out of range (rows=%d V=%d)", rows, V);
  if (K < 1 || K > DDTREE_MAX_TOPK || K > V)
    return fail(DDTREE_EINVAL, "ddtree_draft_topk: K=%d must be in [1, min(V, %d)]", K,
                DDTREE_MAX_TOPK);
  if (rows > 65535)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_draft_topk: %d rows exceed 65535", rows);
  int ept, S, chunk;
  topk_plan(rows, V, &ept, &S, &chunk);
  const size_t need = topk_ws_bytes(rows, S, K);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(DDTREE_EINVAL, "ddtree_draft_topk: workspace of %zu bytes needed, got %zu", need,
                workspace_bytes);
  uint64_t* wk = static_cast<uint64_t*>(workspace);
  float2* wm = need ? reinterpret_cast<float2*>(wk + static_cast<size_t>(rows) * S * K) : nullptr;
  if (dtype == DDTREE_BF16)
    launch_topk<uint16_t>(ept, logits, rows, V, K, S, chunk, wk, wm, tokens, logprobs, stream);
  else
    launch_topk<float>(ept, logits, rows, V, K, S, chunk, wk, wm, tokens, logprobs, stream);
  return check_launch("ddtree_draft_topk");
}
