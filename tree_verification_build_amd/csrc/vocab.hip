// ddtree_vocab_reduce: one pass over the target logits of every tree node.
//
// "Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1 step 4
// (argmax at every node) and Section 3 (softmax at temperature T).
//
// Greedy mode streams each row in S slices: a workgroup of 256 threads reads
// its slice with 16-byte coalesced loads and reduces a packed 64-bit key
// (order-preserving value bits << 32 | ~token id), whose maximum is the
// largest logit at the lowest id; it also keeps a running (max, sum exp) for
// the optional log-sum-exp.  When a row is split (S > 1) each slice stores its
// key (and max, sum) in the workspace and a second, one-wave-per-row kernel
// merges the S slices: a kernel boundary orders the two without device-scope
// atomics, whose round trips and per-row contention cost more than the extra
// launch.  Integer keys make the merge order irrelevant: the argmax is the
// same for any S.
//
// Sampling mode needs the row maximum before any weight can be formed, so one
// 1024-thread workgroup owns a row and keeps it in registers: one HBM read,
// then the max/argmax reduction, then the exact 64-bit sum of the integer
// weights (common.hpp: weight()).
#include <algorithm>

#include "common.hpp"

namespace ddt {

ddtree_status check_tree(const ddtree_tree* t, const char* who);

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSplitThreads = 256;
// blocks of DDTREE_R_BLOCK tokens a sampling row may have (V <= 64 blocks)
constexpr int kMaxRowBlocks = 64;
constexpr int kRowThreads = 1024;

// 16 bytes of logits (E = 8 bf16 or 4 fp32 values): raw bits and their floats.
template <typename T> struct Vec;
template <> struct Vec<uint16_t> {
  static constexpr int E = 8;
  __device__ __forceinline__ static void unpack(const u32x4_t& r, float* v) {
    const u32x4_t w = r;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
  // element-wise gather with -inf (0xFF80) past `lim`
  __device__ __forceinline__ static u32x4_t gather(const uint16_t* row, long i, long lim) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = (i + 2 * k < lim) ? row[i + 2 * k] : 0xFF80u;
      const uint32_t b = (i + 2 * k + 1 < lim) ? row[i + 2 * k + 1] : 0xFF80u;
      w[k] = a | (b << 16);
    }
    return u32x4_t{w[0], w[1], w[2], w[3]};
  }
  static constexpr uint32_t kNegInfWord = 0xFF80FF80u;
};
template <> struct Vec<float> {
  static constexpr int E = 4;
  __device__ __forceinline__ static void unpack(const u32x4_t& r, float* v) {
    v[0] = __uint_as_float(r[0]);
    v[1] = __uint_as_float(r[1]);
    v[2] = __uint_as_float(r[2]);
    v[3] = __uint_as_float(r[3]);
  }
  __device__ __forceinline__ static u32x4_t gather(const float* row, long i, long lim) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = (i + k < lim) ? __float_as_uint(row[i + k]) : 0xFF800000u;
    return u32x4_t{w[0], w[1], w[2], w[3]};
  }
  static constexpr uint32_t kNegInfWord = 0xFF800000u;
};

// Raw 16 bytes of logits starting at index i; elements at or past `lim`
// read as -inf.  `vec` says the row base is 16-byte aligned.
template <typename T>
__device__ __forceinline__ u32x4_t load_raw(const T* row, long i, long lim, bool vec) {
  constexpr int E = Vec<T>::E;
  if (vec && i + E <= lim) return *reinterpret_cast<const u32x4_t*>(row + i);
  if (i >= lim) {
    const uint32_t z = Vec<T>::kNegInfWord;
    return u32x4_t{z, z, z, z};
  }
  return Vec<T>::gather(row, i, lim);
}

template <typename T>
__device__ __forceinline__ void load_e(const T* row, long i, long lim, bool vec, float* v) {
  Vec<T>::unpack(load_raw<T>(row, i, lim, vec), v);
}

__device__ __forceinline__ uint64_t pack_key(float v, int idx) {
  return (static_cast<uint64_t>(ord_f32(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(idx));
}

// Running (max, sum exp(x - max)) merge.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
  } else if (m2 > -__builtin_huge_valf()) {
    s += s2 * __expf(m2 - m);
  }
}

template <typename T, bool kLse>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(
    const T* __restrict__ logits, int N, int V, const int32_t* __restrict__ num_nodes, int S,
    int chunk, uint64_t* __restrict__ ws_key, float2* __restrict__ ws_ms,
    int32_t* __restrict__ argmax, float* __restrict__ maxv,
    float* __restrict__ lse) {
  constexpr int E = Vec<T>::E;
  constexpr int kWaves = kSplitThreads / kWave;
  __shared__ uint64_t s_key[kWaves];
  __shared__ float2 s_ms[kWaves];
  const int row = blockIdx.y;
  const int s = blockIdx.x;
  const int b = row / N, n = row % N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The slice is read whatever num_nodes says (rows of padding nodes exist in
  // memory), so that its loads do not wait for that value; padding rows are
  // discarded afterwards.  U vectors per thread are in flight at a time.
  constexpr int U = 4;
  uint64_t key = 0;
  float m = -__builtin_huge_valf(), sum = 0.0f;
  {
    const T* rp = logits + static_cast<long>(row) * V;
    const bool vec = aligned16(rp);
    const bool fast = vec && V % E == 0;   // every in-range vector is whole (chunk % E == 0)
    const int lo = s * chunk, hi = min(V, lo + chunk);
    for (int i0 = lo + tid * E; i0 < hi; i0 += U * kSplitThreads * E) {
      u32x4_t raw[U];
      if (fast) {
        // whole 16-byte vectors: plain predicated loads, all U in flight
        constexpr uint32_t z = Vec<T>::kNegInfWord;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kSplitThreads * E;
          raw[u] = i < hi ? *reinterpret_cast<const u32x4_t*>(rp + i) : u32x4_t{z, z, z, z};
        }
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = load_raw<T>(rp, i0 + u * kSplitThreads * E, hi, vec);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * kSplitThreads * E;
        float v[E];
        Vec<T>::unpack(raw[u], v);
        float vm = v[0];
        int vi = 0;
#pragma unroll
        for (int k = 1; k < E; ++k)
          if (v[k] > vm) { vm = v[k]; vi = k; }
        const uint64_t kk = i < hi ? pack_key(vm, i + vi) : 0ull;
        key = kk > key ? kk : key;
        if (kLse && i < hi) {
          float es = 0.0f;
          const float mm = max(m, vm);
#pragma unroll
          for (int k = 0; k < E; ++k) es += __expf(v[k] - mm);
          sum = (m > -__builtin_huge_valf() ? sum * __expf(m - mm) : 0.0f) + es;
          m = mm;
        }
      }
    }
  }
  const bool valid = n < num_nodes[b];
  if (!valid) {
    key = 0;
    m = -__builtin_huge_valf();
    sum = 0.0f;
  }
  key = wave_max_u64(key);
  if (kLse) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float m2 = shfl_xor_f32(m, o), s2 = shfl_xor_f32(sum, o);
      lse_merge(m, sum, m2, s2);
    }
  }
  if (lane == 0) {
    s_key[wave] = key;
    s_ms[wave] = make_float2(m, sum);
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kWaves; ++w) {
      key = s_key[w] > key ? s_key[w] : key;
      if (kLse) lse_merge(m, sum, s_ms[w].x, s_ms[w].y);
    }
    if (S == 1) {
      argmax[row] = valid ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key)) : -1;
      maxv[row] = valid ? unord_f32(static_cast<uint32_t>(key >> 32)) : -__builtin_huge_valf();
      if (kLse) lse[row] = valid ? m + __logf(sum) : -__builtin_huge_valf();
    } else {
      // this slice's partial result; finalize_kernel merges the row's slices
      ws_key[static_cast<long>(row) * S + s] = key;
      if (kLse) ws_ms[static_cast<long>(row) * S + s] = make_float2(m, sum);
    }
  }
}

// Merge the S slices of each row (one wave per row): the largest packed key
// gives argmax and max; the (max, sum) pairs give the log-sum-exp.
template <bool kLse>
__global__ __launch_bounds__(kWave) void finalize_kernel(int N, const int32_t* __restrict__ num_nodes,
                                                         int S, const uint64_t* __restrict__ ws_key,
                                                         const float2* __restrict__ ws_ms,
                                                         int32_t* __restrict__ argmax,
                                                         float* __restrict__ maxv,
                                                         float* __restrict__ lse) {
  const int row = blockIdx.x, lane = threadIdx.x;
  uint64_t key = 0;
  float m = -__builtin_huge_valf(), sum = 0.0f;
  for (int k = lane; k < S; k += kWave) {
    const uint64_t kk = ws_key[static_cast<long>(row) * S + k];
    key = kk > key ? kk : key;
    if (kLse) {
      const float2 ms = ws_ms[static_cast<long>(row) * S + k];
      lse_merge(m, sum, ms.x, ms.y);
    }
  }
  key = wave_max_u64(key);
  if (kLse) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      float m2 = shfl_xor_f32(m, o), s2 = shfl_xor_f32(sum, o);
      lse_merge(m, sum, m2, s2);
    }
  }
  if (lane == 0) {
    const bool valid = row % N < num_nodes[row / N];
    argmax[row] = valid ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key)) : -1;
    maxv[row] = valid ? unord_f32(static_cast<uint32_t>(key >> 32)) : -__builtin_huge_valf();
    if (kLse) lse[row] = valid ? m + __logf(sum) : -__builtin_huge_valf();
  }
}

// Sampling mode: one workgroup per row, row held in registers (MAXP 16-byte
// vectors per thread, covering up to MAXP * 1024 * E logits).
template <typename T, int MAXP, bool kLse>
__global__ __launch_bounds__(kRowThreads) void row_kernel(
    const T* __restrict__ logits, int N, int V, const int32_t* __restrict__ num_nodes,
    WeightConsts wc, int32_t* __restrict__ argmax, float* __restrict__ maxv,
    uint64_t* __restrict__ R, uint64_t* __restrict__ Rb, float* __restrict__ lse) {
  constexpr int E = Vec<T>::E;
  constexpr int kWaves = kRowThreads / kWave;
  constexpr int kPassPerBlock = DDTREE_R_BLOCK / (kRowThreads * E);   // passes per weight block
  constexpr bool kTab = sizeof(T) == 2 && !kLse;   // bf16 weights from an LDS table
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;
  __shared__ uint64_t s_tab[kTab ? kTabEntries : 1];
  __shared__ uint64_t s_u[kMaxRowBlocks];
  __shared__ uint64_t s_blk[kMaxRowBlocks][kWaves];
  __shared__ float s_f[kWaves];
  __shared__ uint32_t s_i[kWaves];
  const int row = blockIdx.x;
  const int b = row / N, n = row % N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n >= num_nodes[b]) {
    if (tid == 0) {
      argmax[row] = -1;
      maxv[row] = -__builtin_huge_valf();
      R[row] = 0;
      if (kLse) lse[row] = -__builtin_huge_valf();
    }
    if (Rb)
      for (int k = tid; k < nb; k += kRowThreads) Rb[static_cast<long>(row) * nb + k] = 0;
    return;
  }
  // rows are 16-byte aligned and V is a multiple of E here (checked on the host)
  const T* rp = logits + static_cast<long>(row) * V;
  u32x4_t raw[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    const long i = static_cast<long>(p) * kRowThreads * E + tid * E;
    const uint32_t z = Vec<T>::kNegInfWord;
    raw[p] = i < V ? *reinterpret_cast<const u32x4_t*>(rp + i) : u32x4_t{z, z, z, z};
  }
  // the row maximum as a plain float maximum (one op per element), then the
  // lowest index holding it, searched only by the threads that hold it;
  // float equality treats -0 and +0 alike, as the packed keys of the greedy
  // pass do
  float vmax = -__builtin_huge_valf();
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    float v[E];
    Vec<T>::unpack(raw[p], v);
#pragma unroll
    for (int k = 0; k < E; ++k) vmax = max(vmax, v[k]);
    __builtin_amdgcn_sched_barrier(0);   // one pass at a time: bounds live registers
  }
  float bm = vmax;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bm = max(bm, shfl_xor_f32(bm, o));
  if (lane == 0) s_f[wave] = bm;
  __syncthreads();
  float m = s_f[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) m = max(m, s_f[w]);
  m = m + 0.0f;   // -0 -> +0
  uint32_t first = 0xFFFFFFFFu;
  if (vmax == m) {
#pragma unroll
    for (int p = 0; p < MAXP; ++p) {
      float v[E];
      Vec<T>::unpack(raw[p], v);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        const uint32_t idx = static_cast<uint32_t>(p * kRowThreads * E + tid * E + k);
        first = (v[k] == m && idx < first) ? idx : first;
      }
    }
  }
  first = wave_min_u32(first);
  __syncthreads();
  if (lane == 0) s_i[wave] = first;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kWaves; ++w) first = min(first, s_i[w]);

  // bf16 rows take their weights from a table of weight() in LDS (common.hpp:
  // fill_weight_table); a logit outside its window reads 0 and sets its bit
  // in `miss`, and is weighed with weight() itself at the end of its block.
  WeightTable tb{0u, 0u};
  if constexpr (kTab) {
    tb = fill_weight_table(s_tab, m, wc, tid, kRowThreads);
    __syncthreads();
  }
  uint32_t miss = 0;
  auto tab_weight = [&](uint32_t u, int bit) -> uint64_t {
    bool in;
    const uint64_t wv = table_weight(s_tab, tb, u, in);
    miss |= in ? 0u : 1u << bit;
    return wv;
  };

  // weights, summed per block of DDTREE_R_BLOCK tokens (kPassPerBlock passes):
  // each wave's share of a block goes to LDS, the row total is the sum of
  // the blocks
  uint64_t bsum = 0;
  float esum = 0.0f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    // opaque to the optimiser: stops it from keeping the first pass's
    // unpacked floats alive (160 of them) instead of the packed raw bits
    __asm__ volatile("" : "+v"(raw[p]));
    if constexpr (kTab) {
      const u32x4_t w4 = raw[p];
      const int bit0 = (p % kPassPerBlock) * E;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        bsum += tab_weight(w4[k] & 0xFFFFu, bit0 + 2 * k);
        bsum += tab_weight(w4[k] >> 16, bit0 + 2 * k + 1);
        // four lookups in flight at most (registers: see below)
        if (k & 1) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      float v[E];
      Vec<T>::unpack(raw[p], v);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        bsum += weight(v[k], m, wc);
        if (kLse) esum += __expf(v[k] - m);
        // two elements in flight at most: more interleaving runs the 1024-thread
        // workgroup's 128 registers per lane out and spills weights to scratch
        if (k & 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if ((p + 1) % kPassPerBlock == 0 || p == MAXP - 1) {
      if constexpr (kTab) {
        // the block's logits outside the table, weighed directly (re-read
        // from memory: rare, and it keeps weight() out of the unrolled loop)
        if (__builtin_amdgcn_ballot_w64(miss != 0)) {
          const int p0 = p - p % kPassPerBlock;
#pragma unroll 1
          while (miss) {
            const int j = __builtin_ctz(miss);
            miss &= miss - 1u;
            const long i = static_cast<long>(p0 + j / E) * kRowThreads * E + tid * E + j % E;
            // past the row end: the -inf padding, weight 0
            if (i < V) bsum += weight(__uint_as_float(static_cast<uint32_t>(rp[i]) << 16), m, wc);
          }
        }
        miss = 0;
      }
      const uint64_t ws = wave_sum_u64(bsum);
      if (lane == 0) s_blk[p / kPassPerBlock][wave] = ws;
      bsum = 0;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (kLse) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) esum += shfl_xor_f32(esum, o);
  }
  if (lane == 0) s_f[wave] = esum;
  __syncthreads();
  if (tid < nb) {
    uint64_t bt = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) bt += s_blk[tid][w];
    if (Rb) Rb[static_cast<long>(row) * nb + tid] = bt;
    s_u[tid] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t tot = 0;
    float et = 0.0f;
    for (int k = 0; k < nb; ++k) tot += s_u[k];
    for (int w = 0; w < kWaves; ++w) et += s_f[w];
    argmax[row] = static_cast<int32_t>(first);
    maxv[row] = m;
    R[row] = tot;
    if (kLse) lse[row] = m + __logf(et);
  }
}

// Sampling mode for rows too long for registers: two passes over the row.
template <typename T, bool kLse>
__global__ __launch_bounds__(kRowThreads) void row2_kernel(
    const T* __restrict__ logits, int N, int V, const int32_t* __restrict__ num_nodes,
    WeightConsts wc, int32_t* __restrict__ argmax, float* __restrict__ maxv,
    uint64_t* __restrict__ R, uint64_t* __restrict__ Rb, float* __restrict__ lse) {
  constexpr int E = Vec<T>::E;
  constexpr int kWaves = kRowThreads / kWave;
  constexpr int kPassPerBlock = DDTREE_R_BLOCK / (kRowThreads * E);   // passes per weight block
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;
  __shared__ uint64_t s_u[kMaxRowBlocks > kWaves ? kMaxRowBlocks : kWaves];
  __shared__ uint64_t s_blk[kMaxRowBlocks][kWaves];
  __shared__ float s_f[kWaves];
  const int row = blockIdx.x;
  const int b = row / N, n = row % N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (n >= num_nodes[b]) {
    if (tid == 0) {
      argmax[row] = -1;
      maxv[row] = -__builtin_huge_valf();
      R[row] = 0;
      if (kLse) lse[row] = -__builtin_huge_valf();
    }
    if (Rb)
      for (int k = tid; k < nb; k += kRowThreads) Rb[static_cast<long>(row) * nb + k] = 0;
    return;
  }
  const T* rp = logits + static_cast<long>(row) * V;
  const bool vec = aligned16(rp);
  uint64_t key = 0;
  for (long i = static_cast<long>(tid) * E; i < V; i += kRowThreads * E) {
    float v[E];
    load_e<T>(rp, i, V, vec, v);
#pragma unroll
    for (int k = 0; k < E; ++k) {
      const uint64_t kk = pack_key(v[k], static_cast<int>(i) + k);
      key = kk > key ? kk : key;
    }
  }
  key = wave_max_u64(key);
  if (lane == 0) s_u[wave] = key;
  __syncthreads();
  key = s_u[0];
  for (int w = 1; w < kWaves; ++w) key = s_u[w] > key ? s_u[w] : key;
  const float m = unord_f32(static_cast<uint32_t>(key >> 32));
  __syncthreads();
  // per-block weight sums as in row_kernel, one block of passes at a time
  float esum = 0.0f;
  for (int blk = 0; blk < nb; ++blk) {
    uint64_t bsum = 0;
    for (int p = blk * kPassPerBlock; p < (blk + 1) * kPassPerBlock; ++p) {
      const long i = static_cast<long>(p) * kRowThreads * E + static_cast<long>(tid) * E;
      if (i >= V) break;
      float v[E];
      load_e<T>(rp, i, V, vec, v);
#pragma unroll
      for (int k = 0; k < E; ++k) {
        bsum += weight(v[k], m, wc);
        if (kLse) esum += __expf(v[k] - m);
      }
    }
    const uint64_t ws = wave_sum_u64(bsum);
    if (lane == 0) s_blk[blk][wave] = ws;
  }
  if (kLse) {
    for (int o = 32; o >= 1; o >>= 1) esum += shfl_xor_f32(esum, o);
  }
  if (lane == 0) s_f[wave] = esum;
  __syncthreads();
  if (tid < nb) {
    uint64_t bt = 0;
    for (int w = 0; w < kWaves; ++w) bt += s_blk[tid][w];
    if (Rb) Rb[static_cast<long>(row) * nb + tid] = bt;
    s_u[tid] = bt;
  }
  __syncthreads();
  if (tid == 0) {
    uint64_t tot = 0;
    float et = 0.0f;
    for (int k = 0; k < nb; ++k) tot += s_u[k];
    for (int w = 0; w < kWaves; ++w) et += s_f[w];
    argmax[row] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
    maxv[row] = m;
    R[row] = tot;
    if (kLse) lse[row] = m + __logf(et);
  }
}

// Sampling mode for bf16 rows (no log-sum-exp): every logit leaves HBM once
// and is weighed from registers.  Persistent workgroups of 1024 threads, one
// per CU, take rows r, r + G, r + 2G, ... (G workgroups).  A row is held in
// registers (MAXP 16-byte vectors per thread: vector p of thread t covers
// tokens p * 8192 + 8t .. + 7).  Per row: the row maximum (a float maximum,
// then the lowest index holding it), a table of weight() in LDS for the row's
// window of bf16 patterns, then the weight pass, which, as soon as a vector's
// eight logits are weighed, issues the load of the same vector of the
// workgroup's next row into the same registers: the next row streams in
// while this one is weighed, so HBM stays busy while the CU computes.
//
// Table lookup with packed 16-bit arithmetic, two logits per operation: for
// the magnitude pattern a of a logit (its 15 low bits), off = hi - a wraps
// to >= 0x8000 above the window (weight 0 there), lies in [0, span) inside it
// and in [span, 0x7FFF] below it; min(off, span) is the entry within its
// sign's half of the table (entry span of each half is 0), and the sign bit
// of the pattern, kept in place, adds the negative half's 32768-byte offset.
// Each half of the table: entry 0 is the weight 0 of magnitudes above the
// window (a negative logit below m - 32/c: weight() is 0 there), entries 1 ..
// span the window's patterns from the top down, entry span + 1 a sentinel
// (2^56) that the sums count in their top bits for magnitudes below the
// window; those rare logits are weighed with weight() itself after the pass,
// so every weight is weight()'s own value.  The window spans kPipeTabE
// binades (wider than the other kernels' kTabE: below-window logits cost a
// re-read, above-window ones nothing).
constexpr int kPipeTabE = 26;
constexpr int kPipeSpan = kPipeTabE * 128;
constexpr int kPipeNegEntries = 4096;                         // negative half: byte 32768
constexpr uint64_t kOutside = 1ull << 56;   // sentinel of the below-window entries
constexpr int kPipeTabEntries = kPipeNegEntries + kPipeSpan + 2;
static_assert(kPipeSpan + 2 <= kPipeNegEntries, "each half fits its 32 KB");

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// a - b per 16-bit half, saturating at 0
__device__ __forceinline__ uint32_t pk_sub_sat_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, a),
                                                                    __builtin_bit_cast(u16x2_t, b)));
}
typedef int16_t i16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_i16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(i16x2_t, a),
                                                                __builtin_bit_cast(i16x2_t, b)));
}
__device__ __forceinline__ uint32_t pk_ashr15_i16(uint32_t a) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(i16x2_t, a) >> i16x2_t{15, 15});
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}

// (x & 0xFFFF) * 8 in one operation (the compiler emits a shift and a mask)
__device__ __forceinline__ uint32_t mul_lo16_by8(uint32_t x) {
  uint32_t r;
  asm("v_mad_u32_u16 %0, %1, 8, 0" : "=v"(r) : "v"(x));
  return r;
}

// Wave reductions by DPP row moves and lane reads (with wave_sum_u64_dpp of
// common.hpp): no shuffle-index registers (the row kernel below has none to
// spare).
__device__ __forceinline__ float wave_max_f32_dpp(float x) { return unord_f32(wave_max_u32(ord_f32(x))); }
__device__ __forceinline__ uint32_t wave_min_u32_dpp(uint32_t x) { return ~wave_max_u32(~x); }

template <int MAXP, bool WHOLE>
__global__ __launch_bounds__(kRowThreads) void row_pipe_kernel(
    const uint16_t* __restrict__ logits, int rows, int N, int V,
    const int32_t* __restrict__ num_nodes, WeightConsts wc, int32_t* __restrict__ argmax,
    float* __restrict__ maxv, uint64_t* __restrict__ R, uint64_t* __restrict__ Rb, int heavy,
    uint32_t stagger) {
  constexpr int E = 8;
  constexpr int kWaves = kRowThreads / kWave;
  constexpr int kQ = DDTREE_R_BLOCK / (kRowThreads * E);   // vectors per thread per block
  static_assert(kQ == 4, "four 8192-token vectors per weight block");
  __shared__ uint64_t s_tab[kPipeTabEntries];
  __shared__ uint64_t s_blk[kMaxRowBlocks][kWaves];
  __shared__ float s_f[kWaves], s_f2[kWaves];
  __shared__ uint32_t s_i[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;
  int row = blockIdx.x;
  if (row >= rows) return;
  constexpr uint32_t kNegInf2 = Vec<uint16_t>::kNegInfWord;
  // Loads are unconditional, from addresses that are always inside the
  // logits: a load under a condition becomes a load into other registers
  // plus a copy, and the copy waits for the load.  Vector p of a row past its
  // end (WHOLE false) re-reads the row's last vector and is masked to -inf
  // where it is used; with no next row, every thread loads the logits' first
  // 16 bytes (one cached line, never used) instead of a row.
  // t8: this thread's first token of each vector, redefined opaquely every row
  // so that the compiler computes each vector's offset where it loads it
  // instead of keeping MAXP offsets live across the row loop
  uint32_t t8 = tid * E;
  auto vload = [&](int r, int p, bool real = true) -> u32x4_t {
    if (WHOLE) {
      // a uniform base (row and vector) plus the thread's 32-bit byte offset:
      // scalar-register addressing, no per-vector address arithmetic
      const uint16_t* base = real ? logits + static_cast<long>(r) * V + p * kRowThreads * E : logits;
      const uint32_t off = real ? 2u * t8 : 0u;
      return *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const char*>(base) + off);
    }
    uint32_t i = t8 + static_cast<uint32_t>(p * kRowThreads * E);
    i = min(i, static_cast<uint32_t>(V - E));
    const long off = real ? static_cast<long>(r) * V + i : 0l;
    return *reinterpret_cast<const u32x4_t*>(logits + off);
  };
  auto inrow = [&](int p) { return WHOLE || t8 + static_cast<uint32_t>(p * kRowThreads * E) < static_cast<uint32_t>(V); };
  auto word = [&](const u32x4_t& v, int p, int k) { return inrow(p) ? v[k] : kNegInf2; };
  // The running maximum of a thread's logits: a packed pair of 16-bit
  // patterns, one packed operation per two logits, the largest pattern as a
  // signed 16-bit value (patterns of non-negative bf16 values order as their
  // values do, and negative patterns are negative).  A row with no
  // non-negative pattern takes its maximum from the registers again, below.
  // vec_max folds a vector into it.
  typedef uint32_t MaxAcc;
  auto vec_max = [&](MaxAcc acc, const u32x4_t& v, int p) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc = pk_max_i16(acc, word(v, p, k));
    return acc;
  };
  // back to a float: the largest non-negative pattern, -inf if none
  auto key_to_float = [](MaxAcc acc) {
    const int32_t a = static_cast<int16_t>(acc & 0xFFFFu), b = static_cast<int16_t>(acc >> 16);
    const int32_t pmax = max(a, b);
    return pmax >= 0 ? __uint_as_float(static_cast<uint32_t>(pmax) << 16) : -__builtin_huge_valf();
  };
  constexpr MaxAcc kKeyNegInf = 0x80008000u;   // no logit yet
  u32x4_t raw[MAXP];
  // Workgroups [0, heavy) have one row more than the others.  The others wait
  // `stagger` ticks of the constant-rate clock before their first loads, so
  // that the heavy workgroups' first rows arrive at a larger share of the
  // bandwidth and their extra row starts earlier (only the timing changes).
  if (stagger && static_cast<int>(blockIdx.x) >= heavy) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while (__builtin_amdgcn_s_memrealtime() - t0 < stagger) __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int p = 0; p < MAXP; ++p) raw[p] = vload(row, p);
  // this thread's maximum over its logits of the row in raw: for the first
  // row here, for the next ones during the previous row's weight pass
  MaxAcc vkey = kKeyNegInf;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    vkey = vec_max(vkey, raw[p], p);
    __builtin_amdgcn_sched_barrier(0);   // one vector at a time: bounds live registers
  }
  // the weight pass takes the maximum of the next row's vector p - kLag: kLag
  // vectors of weighing after its load was issued
  constexpr int kLag = MAXP > 6 ? 6 : MAXP - 1;

  for (; row < rows; row += gridDim.x) {
    __asm__ volatile("" : "+v"(t8));
    const int next = row + gridDim.x;
    const bool has_next = next < rows;
    const bool valid = row % N < num_nodes[row / N];
    const uint16_t* rp = logits + static_cast<long>(row) * V;
    // ---- the row maximum (this thread's part: vkey), then the lowest index holding it
    float vmax = key_to_float(vkey);
    const float bm = wave_max_f32_dpp(vmax);
    if (lane == 0) s_f[wave] = bm;
    __syncthreads();
    float m = s_f[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = max(m, s_f[w]);
    if (m == -__builtin_huge_valf()) {
      // no pattern of the row is non-negative (the same for every thread):
      // the maximum is the negative pattern nearest zero, the smallest one as
      // an unsigned 16-bit value, taken from the row in registers
      uint32_t neg = 0xFFFFFFFFu;
#pragma unroll
      for (int p = 0; p < MAXP; ++p) {
#pragma unroll
        for (int k = 0; k < 4; ++k) neg = pk_min_u16(neg, word(raw[p], p, k));
      }
      vmax = __uint_as_float(min(neg & 0xFFFFu, neg >> 16) << 16);
      const float bn = wave_max_f32_dpp(vmax);
      if (lane == 0) s_f2[wave] = bn;
      __syncthreads();
      m = s_f2[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) m = max(m, s_f2[w]);
    }
    m = m + 0.0f;   // -0 -> +0
    // bf16 patterns equal to m as floats: m's own pattern, or either zero when m is 0
    uint32_t first = 0xFFFFFFFFu;
    // (when m is 0, a thread may hold -0 with no non-negative pattern)
    if (vmax == m || m == 0.0f) {
      // patterns equal to m as floats, compared with the zero patterns folded
      // together when m is 0; vectors are tested whole first
      const uint32_t zm = m == 0.0f ? 0x7FFFu : 0xFFFFu;
      const uint32_t mb = (__float_as_uint(m) >> 16) & zm;
#pragma unroll
      for (int p = 0; p < MAXP; ++p) {
        bool any = false;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t w = word(raw[p], p, k);
          any |= (w & zm) == mb || ((w >> 16) & zm) == mb;
        }
        if (any && first == 0xFFFFFFFFu) {
#pragma unroll
          for (int k = E - 1; k >= 0; --k) {
            const uint32_t u = (word(raw[p], p, k >> 1) >> (16 * (k & 1))) & zm;
            first = u == mb ? t8 + static_cast<uint32_t>(p * kRowThreads * E + k) : first;
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    first = wave_min_u32_dpp(first);
    if (lane == 0) s_i[wave] = first;
    // ---- the weight table of this row (both halves; entry span of each is 0)
    const float big = max(fabsf(m), fabsf(m - 32.0f / wc.c));
    const int e_top = static_cast<int>((__float_as_uint(big) >> 23) & 0xFFu);
    const int e_hi = min(e_top, 254), e_lo = max(e_top - kPipeTabE + 1, 1);
    const uint32_t hi = (static_cast<uint32_t>(e_hi) << 7) | 127u;
    const uint32_t span = e_hi >= e_lo ? hi - (static_cast<uint32_t>(e_lo) << 7) + 1u : 0u;
    for (int t = tid; t < 2 * (kPipeSpan + 2); t += kRowThreads) {
      const uint32_t neg = t >= kPipeSpan + 2 ? 1u : 0u;
      const uint32_t off = static_cast<uint32_t>(t) - neg * (kPipeSpan + 2);
      uint64_t wv = off == span + 1u ? kOutside : 0ull;
      if (off >= 1u && off <= span) {
        const float l = __uint_as_float(((neg << 15) | (hi + 1u - off)) << 16);
        // patterns above m occur in no row with this maximum; those whose
        // exponent y falls below -32 weigh 0 (weight()'s own cut-off, computed
        // the same way), skipped by whole waves as the window runs in order
        if (l <= m && (l - m) * wc.c >= -32.0f) wv = weight(l, m, wc);
      }
      s_tab[neg * kPipeNegEntries + off] = wv;
    }
    __syncthreads();
    // ---- weights, per block of DDTREE_R_BLOCK tokens, loading the next row behind them
    const uint32_t top2 = (hi + 1u) * 0x10001u, end2 = (span + 1u) * 0x10001u;
    const uint32_t lo_mag = hi + 1u - span;   // magnitudes below this are below the window
    const unsigned char* tab = reinterpret_cast<const unsigned char*>(s_tab);
    constexpr int kBlocks = (MAXP + kQ - 1) / kQ;
    uint64_t bsum[kBlocks];
    MaxAcc nkey = kKeyNegInf;   // the next row's maximum, as its vectors arrive
    uint32_t missed = 0;   // bit b: a logit of block b lies outside the window
#pragma unroll
    for (int blk = 0; blk < kBlocks; ++blk) {
      uint64_t acc = 0;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        const int p = blk * kQ + q;
        if (p < MAXP) {
          // opaque to the optimiser: keeps it from holding unpacked copies of
          // several vectors at once (the row already takes 4 * MAXP registers)
          __asm__ volatile("" : "+v"(raw[p]));
          // the vector's eight table addresses, then its eight lookups in flight
          // together, then their sum.  Entry index per half: the window entry c
          // (< 4096) plus 4096 for a negative pattern (its sign bit moved to bit
          // 12); byte address = index * 8, taken from each half by one shift
          // (the low half's index is below 2^13, so the high half's index
          // shifted right by 13 has nothing of it in its low three bits).
          uint32_t a[E];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t w = word(raw[p], p, k);
            const uint32_t c2 = pk_min_u16(pk_sub_sat_u16(top2, w & 0x7FFF7FFFu), end2);
            const uint32_t i2 = ((w >> 3) & 0x10001000u) | c2;
            a[2 * k] = mul_lo16_by8(i2);
            a[2 * k + 1] = i2 >> 13;
          }
          uint64_t t[E];
#pragma unroll
          for (int j = 0; j < E; ++j) t[j] = *reinterpret_cast<const uint64_t*>(tab + a[j]);
          acc += ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
          // the sums stay per vector (reassociated across vectors they would
          // keep every lookup of the block live at once)
          __asm__ volatile("" : "+v"(acc));
          // this vector is weighed: its registers take the next row's vector
          raw[p] = vload(next, p, has_next);
          if (p >= kLag) {
            nkey = vec_max(nkey, raw[p - kLag], p - kLag);
            // pinned here (the compiler would otherwise sink it to the next
            // row's start, where the loads would be waited for with no work)
            __asm__ volatile("" : "+v"(nkey));
          }
        }
      }
      missed |= acc >= kOutside ? 1u << blk : 0u;
      bsum[blk] = acc & (kOutside - 1u);
    }
#pragma unroll
    for (int p = MAXP - kLag; p < MAXP; ++p) nkey = vec_max(nkey, raw[p], p);
    vkey = nkey;
    // logits below the window (rare): weighed with weight() after the whole
    // pass, from their block's vectors re-read from memory (so that no load of
    // the stream waits for them), one vector at a time
    if (__builtin_amdgcn_ballot_w64(missed != 0)) {
#pragma unroll
      for (int blk = 0; blk < kBlocks; ++blk) {
        if (missed & (1u << blk)) {
#pragma unroll 1
          for (int q = 0; q < kQ; ++q) {
            const int p = blk * kQ + q;
            if (p < MAXP) {
              const u32x4_t v = vload(row, p);
              uint64_t fix = 0;
#pragma unroll
              for (int k = 0; k < E; ++k) {
                const uint32_t u = (word(v, p, k >> 1) >> (16 * (k & 1))) & 0xFFFFu;
                const uint64_t wk = weight(__uint_as_float(u << 16), m, wc);
                fix += (u & 0x7FFFu) < lo_mag ? wk : 0ull;
              }
              bsum[blk] += fix;
            }
          }
        }
      }
    }
#pragma unroll
    for (int blk = 0; blk < kBlocks; ++blk) {
      const uint64_t ws = wave_sum_u64_dpp(bsum[blk]);
      if (lane == 0 && blk < nb) s_blk[blk][wave] = ws;
    }
    __syncthreads();
    if (wave == 0) {
      uint64_t bt = 0;
      if (lane < nb) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) bt += s_blk[lane][w];
        if (Rb) Rb[static_cast<long>(row) * nb + lane] = valid ? bt : 0ull;
      }
      const uint64_t tot = wave_sum_u64_dpp(bt);
      // the lowest index holding the maximum over the waves (read here, not
      // before the weight pass, where the values would stay live through it)
#pragma unroll
      for (int w = 0; w < kWaves; ++w) first = min(first, s_i[w]);
      if (lane == 0) {
        R[row] = valid ? tot : 0ull;
        argmax[row] = valid ? static_cast<int32_t>(first) : -1;
        maxv[row] = valid ? m : -__builtin_huge_valf();
      }
    }
  }
}

// Workgroups of the persistent sampling kernel: one per CU of the device
// (looked up once per device).
int device_cus() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

// The late start of the workgroups with one row fewer, in ticks of the
// device's constant-rate clock: 3 us, measured best on the sampling passes
// of 528 and 2112 rows of 163,840 tokens (2 and 8 whole rounds of 256
// workgroups plus 16 and 64 rows; 2-5 us tried).  Looked up once per device.
constexpr double kStaggerUs = 3.0;
uint32_t stagger_ticks() {
  static uint32_t cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  uint32_t v = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
  if (v == 0) {
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      khz = 100000;   // 100 MHz
    v = static_cast<uint32_t>(kStaggerUs * 1e-3 * khz + 0.5);
    __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
  }
  return v;
}

template <int MAXP>
void launch_pipe(int rows, hipStream_t st, const void* logits, int N, int V, const int32_t* nn,
                 const WeightConsts& wc, int32_t* am, float* mx, uint64_t* R, uint64_t* Rb) {
  const int G = std::min(rows, device_cus());
  // rows = F * G + heavy: with 0 < heavy, the other workgroups start late
  const int heavy = rows % G;
  const uint32_t stagger = heavy ? stagger_ticks() : 0u;
  if (V == MAXP * kRowThreads * 8)
    hipLaunchKernelGGL((row_pipe_kernel<MAXP, true>), dim3(G), dim3(kRowThreads), 0, st,
                       static_cast<const uint16_t*>(logits), rows, N, V, nn, wc, am, mx, R, Rb,
                       heavy, stagger);
  else
    hipLaunchKernelGGL((row_pipe_kernel<MAXP, false>), dim3(G), dim3(kRowThreads), 0, st,
                       static_cast<const uint16_t*>(logits), rows, N, V, nn, wc, am, mx, R, Rb,
                       heavy, stagger);
}

// true when launched: bf16 rows of whole 16-byte vectors, up to 20 of them per
// thread; rows that end inside a vector past the eighth (whose masking would
// not fit the 128 registers) take the row-per-workgroup kernel instead
bool launch_sampling_pipe(int rows, hipStream_t st, const void* logits, int N, int V,
                          const int32_t* nn, const WeightConsts& wc, int32_t* am, float* mx,
                          uint64_t* R, uint64_t* Rb) {
  if (V % 8 != 0 || !aligned16(logits)) return false;
  const int passes = (V + kRowThreads * 8 - 1) / (kRowThreads * 8);
  if (passes > 8 && V % (kRowThreads * 8) != 0) return false;
  if (passes <= 1) launch_pipe<1>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 2) launch_pipe<2>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 4) launch_pipe<4>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 8) launch_pipe<8>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 12) launch_pipe<12>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 16) launch_pipe<16>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else if (passes <= 20) launch_pipe<20>(rows, st, logits, N, V, nn, wc, am, mx, R, Rb);
  else return false;
  return true;
}

// Greedy merge and walk in one launch: one workgroup per request merges the
// slice keys of all its rows (an LDS 64-bit maximum per row: the largest
// packed key, as in finalize_kernel, hence the same argmax and max), writes
// argmax and max, and its first wave then walks the tree from LDS
// (common.hpp: walk_run).  The dependent launch this saves is most of the
// cost of the merge and of the walk at small batch.
constexpr int kMergeWalkThreads = 1024;

__global__ __launch_bounds__(kMergeWalkThreads) void merge_walk_kernel(
    ddtree_tree t, int S, const uint64_t* __restrict__ ws_key, int32_t* __restrict__ argmax,
    float* __restrict__ maxv, int32_t* __restrict__ accept_len, int32_t* __restrict__ path_nodes,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ bonus) {
  __shared__ unsigned long long s_key[DDTREE_MAX_NODES];
  __shared__ int32_t s_am[DDTREE_MAX_NODES];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = t.N;
  const long base = static_cast<long>(b) * N;
  WalkNodes w{};
  if (wave == 0) w = walk_load(t, b, lane);
  for (int n = tid; n < N; n += kMergeWalkThreads) s_key[n] = 0ull;
  const int nn = t.num_nodes[b];
  __syncthreads();
  // this request's keys: S per row, rows base .. base + N - 1; four loads in
  // flight per thread before their LDS maxima
  const uint64_t* keys = ws_key + base * S;
  const int total = N * S;
  for (int i0 = tid; i0 < total; i0 += 4 * kMergeWalkThreads) {
    uint64_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kMergeWalkThreads;
      kk[u] = i < total ? keys[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * kMergeWalkThreads;
      if (i < total) atomicMax(&s_key[i / S], static_cast<unsigned long long>(kk[u]));
    }
  }
  __syncthreads();
  for (int n = tid; n < N; n += kMergeWalkThreads) {
    const bool valid = n < nn;
    const uint64_t key = s_key[n];
    const int am = valid ? static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key)) : -1;
    argmax[base + n] = am;
    maxv[base + n] = valid ? unord_f32(static_cast<uint32_t>(key >> 32)) : -__builtin_huge_valf();
    s_am[n] = am;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const bool ok = lane + s2 * kWave < nn;
      w.par[s2] = ok ? w.par[s2] : -2;
      w.tok[s2] = ok ? w.tok[s2] : -2;
    }
    walk_run(t, b, s_am, w, lane, accept_len, path_nodes, out_tokens, bonus);
  }
}

// Split count for the greedy pass: enough workgroups to cover the chip
// (about 1024 resident), each slice a whole number of 16-byte vectors per thread.
void split_plan(int rows, int V, int elem_bytes, int* S_out, int* chunk_out) {
  const int per_pass = kSplitThreads * (16 / elem_bytes);
  int S = std::max(1, std::min((1024 + rows - 1) / rows, (V + per_pass - 1) / per_pass));
  int chunk = (V + S - 1) / S;
  chunk = (chunk + per_pass - 1) / per_pass * per_pass;
  // a slice of more than four passes is cut to whole multiples of four, so that
  // every thread's loads go out in one batch (split_kernel keeps four 16-byte
  // vectors in flight): long's 65 rows, 10240 -> 8192 tokens per slice
  constexpr int kRound = 4;
  if (chunk > kRound * per_pass) chunk = chunk / (kRound * per_pass) * (kRound * per_pass);
  S = (V + chunk - 1) / chunk;
  *S_out = S;
  *chunk_out = chunk;
}

template <typename T, int MAXP>
void launch_row(dim3 grid, hipStream_t st, const void* logits, int N, int V, const int32_t* nn,
                const WeightConsts& wc, int32_t* am, float* mx, uint64_t* R, uint64_t* Rb,
                float* lse) {
  if (lse)
    hipLaunchKernelGGL((row_kernel<T, MAXP, true>), grid, dim3(kRowThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
  else
    hipLaunchKernelGGL((row_kernel<T, MAXP, false>), grid, dim3(kRowThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
}

template <typename T>
void launch_sampling(int rows, hipStream_t st, const void* logits, int N, int V,
                     const int32_t* nn, const WeightConsts& wc, int32_t* am, float* mx,
                     uint64_t* R, uint64_t* Rb, float* lse) {
  const int per_pass = kRowThreads * Vec<T>::E;
  const int passes = (V + per_pass - 1) / per_pass;
  const bool fits = V % Vec<T>::E == 0 && aligned16(logits);
  const dim3 g(rows);
  if (!fits) {
    if (lse)
      hipLaunchKernelGGL((row2_kernel<T, true>), g, dim3(kRowThreads), 0, st,
                         static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
    else
      hipLaunchKernelGGL((row2_kernel<T, false>), g, dim3(kRowThreads), 0, st,
                         static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
  } else if (passes <= 1) launch_row<T, 1>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 2) launch_row<T, 2>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 4) launch_row<T, 4>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 8) launch_row<T, 8>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 12) launch_row<T, 12>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 16) launch_row<T, 16>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (passes <= 20) launch_row<T, 20>(g, st, logits, N, V, nn, wc, am, mx, R, Rb, lse);
  else if (lse)
    hipLaunchKernelGGL((row2_kernel<T, true>), g, dim3(kRowThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
  else
    hipLaunchKernelGGL((row2_kernel<T, false>), g, dim3(kRowThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, wc, am, mx, R, Rb, lse);
}

// Greedy workspace: [rows * S] uint64 slice keys, then [rows * S] float2
// (max, sum) slice partials; no initialisation needed.
size_t greedy_ws_bytes(int rows, int S) {
  if (S <= 1) return 0;
  return static_cast<size_t>(rows) * S * (sizeof(uint64_t) + sizeof(float2));
}

template <typename T>
void launch_greedy(int rows, int N, int V, hipStream_t st, const void* logits, const int32_t* nn,
                   int S, int chunk, void* ws, int32_t* am, float* mx, float* lse,
                   bool merge = true) {
  uint64_t* ws_key = static_cast<uint64_t*>(ws);
  float2* ws_ms = reinterpret_cast<float2*>(ws_key + static_cast<size_t>(rows) * S);
  const dim3 grid(S, rows);
  if (lse)
    hipLaunchKernelGGL((split_kernel<T, true>), grid, dim3(kSplitThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, S, chunk, ws_key, ws_ms, am, mx,
                       lse);
  else
    hipLaunchKernelGGL((split_kernel<T, false>), grid, dim3(kSplitThreads), 0, st,
                       static_cast<const T*>(logits), N, V, nn, S, chunk, ws_key, ws_ms, am, mx,
                       lse);
  if (S > 1 && merge) {
    if (lse)
      hipLaunchKernelGGL((finalize_kernel<true>), dim3(rows), dim3(kWave), 0, st, N, nn, S, ws_key,
                         ws_ms, am, mx, lse);
    else
      hipLaunchKernelGGL((finalize_kernel<false>), dim3(rows), dim3(kWave), 0, st, N, nn, S, ws_key,
                         ws_ms, am, mx, lse);
  }
}

}  // namespace
}  // namespace ddt

extern "C" size_t ddtree_vocab_reduce_workspace_size(int32_t B, int32_t N, int32_t V) {
  if (B < 1 || N < 1 || V < 1) return 0;
  int S2, S4, chunk;
  ddt::split_plan(B * N, V, 2, &S2, &chunk);
  ddt::split_plan(B * N, V, 4, &S4, &chunk);
  const int S = S2 > S4 ? S2 : S4;               // covers both element sizes
  return ddt::greedy_ws_bytes(B * N, S);
}

extern "C" ddtree_status ddtree_vocab_reduce(const void* logits, ddtree_dtype dtype, int32_t B,
                                             int32_t N, int32_t V, const int32_t* num_nodes,
                                             float temperature, int32_t* argmax, float* maxv,
                                             uint64_t* R, uint64_t* R_blocks, float* lse,
                                             void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  using namespace ddt;
  if (!logits || !num_nodes || !argmax || !maxv)
    return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: null pointer");
  if (B < 1 || N < 1 || N > DDTREE_MAX_NODES || V < 1)
    return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: sizes out of range (B=%d N=%d V=%d)", B, N, V);
  if (!(temperature >= 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: temperature must be >= 0 and finite");
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: unknown dtype %d", static_cast<int>(dtype));
  const int rows = B * N;
  if (temperature > 0.0f) {
    if (!R) return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: R is required when temperature > 0");
    if (V > kMaxRowBlocks * DDTREE_R_BLOCK)
      return fail(DDTREE_EUNSUPPORTED, "ddtree_vocab_reduce: V = %d exceeds %d for sampling", V,
                  kMaxRowBlocks * DDTREE_R_BLOCK);
    const WeightConsts wc = weight_consts(temperature);
    // bf16 rows without the log-sum-exp: one pass over HBM, rows pipelined
    // through registers (row_pipe_kernel); otherwise a workgroup per row
    const bool piped = dtype == DDTREE_BF16 && !lse &&
                       launch_sampling_pipe(rows, stream, logits, N, V, num_nodes, wc, argmax,
                                            maxv, R, R_blocks);
    if (piped) {
      // launched
    } else if (dtype == DDTREE_BF16) {
      launch_sampling<uint16_t>(rows, stream, logits, N, V, num_nodes, wc, argmax, maxv, R,
                                R_blocks, lse);
    } else {
      launch_sampling<float>(rows, stream, logits, N, V, num_nodes, wc, argmax, maxv, R, R_blocks,
                             lse);
    }
    return check_launch("ddtree_vocab_reduce");
  }
  int S, chunk;
  split_plan(rows, V, dtype == DDTREE_BF16 ? 2 : 4, &S, &chunk);
  if (S > 1) {
    const size_t need = greedy_ws_bytes(rows, S);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
      return fail(DDTREE_EINVAL, "ddtree_vocab_reduce: workspace of %zu bytes needed, got %zu",
                  need, workspace_bytes);
  }
  if (dtype == DDTREE_BF16)
    launch_greedy<uint16_t>(rows, N, V, stream, logits, num_nodes, S, chunk, workspace, argmax,
                            maxv, lse);
  else
    launch_greedy<float>(rows, N, V, stream, logits, num_nodes, S, chunk, workspace, argmax,
                         maxv, lse);
  return check_launch("ddtree_vocab_reduce");
}

extern "C" ddtree_status ddtree_vocab_verify_greedy(const void* logits, ddtree_dtype dtype,
                                                    int32_t V, const ddtree_tree* tree,
                                                    int32_t* argmax, float* maxv,
                                                    int32_t* accept_len, int32_t* path_nodes,
                                                    int32_t* out_tokens, int32_t* bonus,
                                                    void* workspace, size_t workspace_bytes,
                                                    hipStream_t stream) {
  using namespace ddt;
  const char* who = "ddtree_vocab_verify_greedy";
  if (const ddtree_status st = check_tree(tree, who)) return st;
  if (!logits || !argmax || !maxv || !accept_len || !path_nodes || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "%s: null pointer", who);
  if (V < 1) return fail(DDTREE_EINVAL, "%s: V = %d", who, V);
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "%s: unknown dtype %d", who, static_cast<int>(dtype));
  const int rows = tree->B * tree->N;
  int S, chunk;
  split_plan(rows, V, dtype == DDTREE_BF16 ? 2 : 4, &S, &chunk);
  if (S > 1) {
    const size_t need = greedy_ws_bytes(rows, S);
    if (!workspace || workspace_bytes < need || !aligned16(workspace))
      return fail(DDTREE_EINVAL, "%s: workspace of %zu bytes needed, got %zu", who, need,
                  workspace_bytes);
  }
  uint64_t* ws_key = static_cast<uint64_t*>(workspace);
  float2* ws_ms = reinterpret_cast<float2*>(ws_key + static_cast<size_t>(rows) * S);
  const dim3 grid(S, rows);
  if (dtype == DDTREE_BF16)
    hipLaunchKernelGGL((split_kernel<uint16_t, false>), grid, dim3(kSplitThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), tree->N, V, tree->num_nodes, S, chunk,
                       ws_key, ws_ms, argmax, maxv, nullptr);
  else
    hipLaunchKernelGGL((split_kernel<float, false>), grid, dim3(kSplitThreads), 0, stream,
                       static_cast<const float*>(logits), tree->N, V, tree->num_nodes, S, chunk,
                       ws_key, ws_ms, argmax, maxv, nullptr);
  if (S == 1)   // the split pass wrote argmax and max itself: the plain walk follows
    return ddtree_verify_greedy(tree, argmax, accept_len, path_nodes, out_tokens, bonus, stream);
  hipLaunchKernelGGL(merge_walk_kernel, dim3(tree->B), dim3(kMergeWalkThreads), 0, stream, *tree,
                     S, ws_key, argmax, maxv, accept_len, path_nodes, out_tokens, bonus);
  return check_launch(who);
}
