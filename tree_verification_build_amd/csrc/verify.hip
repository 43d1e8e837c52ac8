// ddtree_verify_greedy / ddtree_verify_sample: verified-tree walks.
//
// Greedy ("Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
// step 5): one wavefront per request.  Every lane holds two nodes; a step of
// the walk is one ballot over "parent == cur and token == argmax[cur]".
//
// Sampled (same page, Section 3; "Implementing Temperature-Aware Tree
// Sampling for DDTree", "Path B"): one 1024-thread workgroup per request.
// The workgroup first gathers, in parallel, the weight every node's token has
// under its parent's target row; wave 0 walks the tree with exact integer
// draws (t = mulhi(u, R_res); accept iff t < w).  Where the walk stops, the
// residual draw finds its 32768-token block from the row's block sums (the
// rejected tokens' weights taken off their blocks), the whole workgroup
// weighs that block, and an exact integer prefix scan picks the bonus token.
//
// Every walk stores accept_len last: each wave that wrote outputs releases
// them at system scope, then one thread releases again and stores accept_len,
// so a host polling accept_len in mapped host memory finds the rest written.
#include "common.hpp"

namespace ddt {

ddtree_status check_tree(const ddtree_tree* t, const char* who);

namespace {

constexpr int kMaxN = DDTREE_MAX_NODES;

__global__ __launch_bounds__(64) void greedy_kernel(ddtree_tree t, const int32_t* __restrict__ argmax,
                                                    int32_t* __restrict__ accept_len,
                                                    int32_t* __restrict__ path_nodes,
                                                    int32_t* __restrict__ out_tokens,
                                                    int32_t* __restrict__ bonus) {
  __shared__ int32_t s_am[kMaxN];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = t.N;
  const long base = static_cast<long>(b) * N;
  // the tree and argmax rows are read before num_nodes is known (all N
  // entries exist), so that the loads do not wait for it
  WalkNodes w = walk_load(t, b, lane);
  int am[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + s * kWave;
    am[s] = j < N ? argmax[base + j] : -1;
  }
  const int nn = t.num_nodes[b];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + s * kWave;
    const bool ok = j < nn;
    w.par[s] = ok ? w.par[s] : -2;
    w.tok[s] = ok ? w.tok[s] : -2;
    if (j < N) s_am[j] = ok ? am[s] : -1;
  }
  __syncthreads();
  walk_run(t, b, s_am, w, lane, accept_len, path_nodes, out_tokens, bonus);
}

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 32 consecutive tokens of a row, as floats (16-byte loads when the row is
// aligned and whole, element loads otherwise); tokens past V read as -inf
template <typename T>
__device__ __forceinline__ void load32(const T* row, long x0, int V, float (&v)[32]) {
  constexpr int P = Elem<T>::kPer16;   // elements per 16 bytes
  if (aligned16(row + x0) && x0 + 32 <= V) {
#pragma unroll
    for (int q = 0; q < 32 / P; ++q) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + x0 + q * P);
#pragma unroll
      for (int e = 0; e < P; ++e) {
        if (P == 8) v[q * P + e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
        else v[q * P + e] = __uint_as_float(w[e]);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e)
      v[e] = x0 + e < V ? Elem<T>::get(row, x0 + e) : -__builtin_huge_valf();
  }
}

constexpr int kTokPerThread = DDTREE_R_BLOCK / kSampleThreads;
static_assert(kTokPerThread == 32, "one weight block = 32 tokens per thread");

// Top-p: a token is in its row's nucleus iff its weight exceeds the row's
// threshold weight, or equals it and its id is at most the threshold id.
__device__ __forceinline__ bool in_nucleus(uint64_t w, long x, uint64_t tw, int ti) {
  return w > tw || (w == tw && x <= ti);
}

// NUC: the walk runs on the rows' top-p nuclei (R and Rb are then the kept
// totals and block sums, thr_w / thr_id the rows' thresholds).
template <typename T, bool NUC>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    ddtree_tree t, const T* __restrict__ logits, int V, const float* __restrict__ maxv,
    const uint64_t* __restrict__ R, const uint64_t* __restrict__ Rb, WeightConsts wc,
    const uint64_t* __restrict__ uniforms, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path_nodes, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ bonus, const uint64_t* __restrict__ thr_w,
    const int32_t* __restrict__ thr_id) {
  __shared__ uint64_t s_w[kMaxN], s_R[kMaxN], s_u0[kMaxN], s_u1[kMaxN];
  __shared__ int32_t s_tok[kMaxN], s_fc[kMaxN], s_ns[kMaxN];
  __shared__ int32_t s_rej[DDTREE_MAX_TOPK];
  __shared__ uint64_t s_wave[kSampleWaves];
  __shared__ int s_nrej, s_cur, s_a, s_blk;
  __shared__ uint64_t s_trem;
  __shared__ uint64_t s_tab[sizeof(T) == 2 ? kTabEntries : 1];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int N = t.N, D = t.D;
  const long base = static_cast<long>(b) * N;
  const int nn = t.num_nodes[b];
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;

  // every node's token, links, totals, uniforms and the weight of its token
  // under its parent's row, one thread per node
  for (int j = tid; j < N; j += kSampleThreads) {
    uint64_t w = 0;
    int tk = -1, fc = -1, ns = -1;
    if (j < nn) {
      tk = t.token[base + j];
      fc = t.first_child[base + j];
      ns = t.next_sibling[base + j];
      if (j > 0 && tk >= 0 && tk < V) {
        const int p = t.parent[base + j];
        const float l = Elem<T>::get(logits, (base + p) * static_cast<long>(V) + tk);
        w = weight(l, maxv[base + p], wc);
        if constexpr (NUC) {
          if (!in_nucleus(w, tk, thr_w[base + p], thr_id[base + p])) w = 0;
        }
      }
    }
    s_w[j] = w;
    s_tok[j] = tk;
    s_fc[j] = fc;
    s_ns[j] = ns;
    s_R[j] = R[base + j];
    s_u0[j] = uniforms[(base + j) * 2 + 0];
    s_u1[j] = uniforms[(base + j) * 2 + 1];
  }
  __syncthreads();

  if (wave == 0) {
    // the walk (every lane follows the same uniform path); both loops are
    // capped (depth <= D, children <= K), so a malformed tree cannot hang
    int32_t* path = path_nodes + static_cast<long>(b) * (D + 1);
    int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
    int cur = 0, a = 0, nrej = 0;
    uint64_t rres = 0;
    while (true) {
      rres = s_R[cur];
      nrej = 0;
      int c = s_fc[cur];
      bool moved = false;
      while (c >= 0 && c < N && nrej < t.K) {
        const uint64_t wcur = s_w[c];
        if (__umul64hi(s_u0[c], rres) < wcur) {
          moved = true;
          break;
        }
        rres -= wcur;
        if (lane == 0) s_rej[nrej] = s_tok[c];
        ++nrej;
        c = s_ns[c];
      }
      if (!moved || a >= D) break;
      if (lane == 0) outt[a] = s_tok[c];
      cur = c;
      ++a;
      if (lane == 0) path[a] = c;
    }
    // residual draw: which weight block holds it (the rejected tokens'
    // weights come off their blocks), one block per lane
    const uint64_t tdraw = __umul64hi(s_u1[cur], rres);
    uint64_t bs = 0;   // nb <= 64 (checked on the host)
    if (lane < nb) {
      bs = Rb[(base + cur) * nb + lane];
      int c = s_fc[cur];
      for (int r = 0; r < nrej && c >= 0; ++r) {   // the rejected children, in order
        if (s_tok[c] / DDTREE_R_BLOCK == lane) bs -= s_w[c];
        c = s_ns[c];
      }
    }
    const uint64_t incl = wave_incl_scan_u64(bs, lane);
    const uint64_t hit = __ballot(lane < nb && incl > tdraw);
    const int blk = hit ? __builtin_ctzll(hit) : nb - 1;
    const uint64_t ex = incl - bs;
    const uint32_t exl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex), blk));
    const uint32_t exh = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex >> 32), blk));
    if (lane == 0) {
      path[0] = 0;
      s_nrej = nrej;
      s_cur = cur;
      s_a = a;
      s_blk = blk;
      s_trem = tdraw - ((static_cast<uint64_t>(exh) << 32) | exl);
    }
    for (int k = a + 1 + lane; k <= D; k += kWave) {
      path[k] = -1;
      outt[k] = -1;
    }
  }
  __syncthreads();

  // within the block: 32 consecutive tokens per thread, an exclusive scan of
  // the per-thread sums in token order, then the thread holding the draw
  // walks its tokens
  const int cur = s_cur, nrej = s_nrej;
  const uint64_t trem = s_trem;
  const float m = maxv[base + cur];
  const uint64_t tw = NUC ? thr_w[base + cur] : 0;
  const int ti = NUC ? thr_id[base + cur] : 0;
  const T* row = logits + (base + cur) * static_cast<long>(V);
  const long x0 = static_cast<long>(s_blk) * DDTREE_R_BLOCK + static_cast<long>(tid) * kTokPerThread;
  float v[32];
  load32<T>(row, x0, V, v);
  // bf16: the row's weights from a table of weight() (common.hpp), filled
  // while the block's logits are in flight; a logit outside the table's
  // window is weighed with weight() itself
  WeightTable tb{0u, 0u};
  if constexpr (sizeof(T) == 2) {
    tb = fill_weight_table(s_tab, m, wc, tid, kSampleThreads);
    __syncthreads();
  }
  auto wt = [&](float l, long x) -> uint64_t {
    uint64_t w;
    if constexpr (sizeof(T) == 2) {
      bool in;
      w = table_weight(s_tab, tb, __float_as_uint(l) >> 16, in);
      if (!in) w = weight(l, m, wc);
    } else {
      w = weight(l, m, wc);
    }
    if constexpr (NUC) return in_nucleus(w, x, tw, ti) ? w : 0;
    return w;
  };
  uint64_t sum = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) sum += wt(v[e], x0 + e);   // -inf past V weighs 0
  for (int r = 0; r < nrej; ++r) {
    const long x = s_rej[r];
    if (x >= x0 && x < x0 + 32) sum -= wt(v[x - x0], x);   // rejected: excluded
  }
  const uint64_t incl = wave_incl_scan_u64(sum, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int k = 0; k < wave; ++k) before += s_wave[k];
  const uint64_t excl = before + incl - sum;
  // The wave holding the draw finds it: lane e takes token e of the thread
  // whose range contains the draw (shuffled from that thread's registers),
  // weighs it (0 when rejected), and an inclusive scan of the 32 weights
  // gives the first token whose running sum passes the draw.
  const uint64_t holder = __ballot(excl <= trem && trem < excl + sum);
  if (holder) {
    const int src = __builtin_ctzll(holder);
    const uint64_t excl_s = __shfl(excl, src, kWave);
    float x = -__builtin_huge_valf();
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float t = __shfl(v[e], src, kWave);
      x = lane == e ? t : x;
    }
    const long xs = static_cast<long>(s_blk) * DDTREE_R_BLOCK +
                    static_cast<long>(wave * kWave + src) * kTokPerThread + lane;
    bool rej = false;
    for (int r = 0; r < nrej; ++r) rej |= (s_rej[r] == xs);
    const uint64_t w = lane < 32 && !rej ? wt(x, xs) : 0ull;
    const uint64_t incl_s = wave_incl_scan_u64(w, lane);
    const uint64_t hit = __ballot(lane < 32 && excl_s + incl_s > trem);
    if (lane == 0) {
      const int pick = hit ? static_cast<int>(xs) + __builtin_ctzll(hit) : -1;
      int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
      outt[s_a] = pick;
      bonus[b] = pick;
    }
    // this wave's stores complete and visible before the barrier below (a
    // workgroup barrier alone does not wait for another wave's stores)
    release_system();
  }
  // accept_len last, after every wave's outputs and a system-scope release:
  // a host that polls it in mapped host memory finds the other outputs written
  __syncthreads();
  if (tid == 0) {
    release_system();
    accept_len[b] = s_a;
  }
}

// ------------------------------------------------------------------ lazy sampled walk
// The same walk as sample_kernel, but the target rows are reduced only when
// the walk reaches them ("Implementing Temperature-Aware Tree Sampling for
// DDTree", "Path B": the softmax only for the visited nodes): for
// the row of the current node the workgroup computes the maximum, then the
// integer weights summed per DDTREE_R_BLOCK block (hence R), with the same
// arithmetic as ddtree_vocab_reduce, so the result is bit-identical to the
// vocab pass followed by sample_kernel.  A row costs one read for the
// maximum and one (mostly from cache) for the weights.
constexpr int kLazyMaxBlocks = 64;

// 16 bytes of logits as floats: E = 8 (bf16) or 4 (fp32); past V reads -inf
template <typename T>
__device__ __forceinline__ void lazy_load16(const T* row, long i, int V, bool vec, float* v) {
  constexpr int E = Elem<T>::kPer16;
  if (vec && i + E <= V) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + i);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (E == 8) v[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
      else v[e] = __uint_as_float(w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = i + e < V ? Elem<T>::get(row, i + e) : -__builtin_huge_valf();
  }
}

// loads in flight per thread in the lazy walk's maximum pass
constexpr int kLazyU = 4;

// 16 bytes of -inf (past the row end) and the floats of 16 raw bytes
template <typename T>
__device__ __forceinline__ u32x4_t lazy_neg_inf() {
  const uint32_t z = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;
  return u32x4_t{z, z, z, z};
}
template <typename T>
__device__ __forceinline__ void lazy_unpack(const u32x4_t& w, float* v) {
  constexpr int E = Elem<T>::kPer16;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (E == 8) v[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
    else v[e] = __uint_as_float(w[e]);
  }
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_lazy_kernel(
    ddtree_tree t, const T* __restrict__ logits, int V, WeightConsts wc,
    const uint64_t* __restrict__ uniforms, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ path_nodes, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ bonus) {
  constexpr int E = Elem<T>::kPer16;
  constexpr int kPass = kSampleThreads * E;                  // tokens per pass
  constexpr int kPassPerBlock = DDTREE_R_BLOCK / kPass;
  static_assert(DDTREE_R_BLOCK % kPass == 0, "passes tile the weight blocks");
  __shared__ uint64_t s_u0[kMaxN], s_u1[kMaxN];
  __shared__ int32_t s_tok[kMaxN], s_fc[kMaxN], s_ns[kMaxN];
  __shared__ int32_t s_rej[DDTREE_MAX_TOPK];
  __shared__ uint64_t s_blkw[kLazyMaxBlocks][kSampleWaves];
  __shared__ uint64_t s_Rb[kLazyMaxBlocks];
  __shared__ uint64_t s_wave[kSampleWaves];
  __shared__ float s_f[kSampleWaves];
  __shared__ int s_nrej, s_cur, s_a, s_go, s_blk;
  __shared__ uint64_t s_rres, s_trem;
  __shared__ uint64_t s_tab[sizeof(T) == 2 ? kTabEntries : 1];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int N = t.N, D = t.D;
  const long base = static_cast<long>(b) * N;
  const int nn = t.num_nodes[b];
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;
  const int npass = (V + kPass - 1) / kPass;

  for (int j = tid; j < N; j += kSampleThreads) {
    int tk = -1, fc = -1, ns = -1;
    if (j < nn) {
      tk = t.token[base + j];
      fc = t.first_child[base + j];
      ns = t.next_sibling[base + j];
    }
    s_tok[j] = tk;
    s_fc[j] = fc;
    s_ns[j] = ns;
    s_u0[j] = uniforms[(base + j) * 2 + 0];
    s_u1[j] = uniforms[(base + j) * 2 + 1];
  }
  if (tid == 0) {
    s_cur = 0;
    s_a = 0;
  }
  __syncthreads();
  int32_t* path = path_nodes + static_cast<long>(b) * (D + 1);
  int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);

  float m = 0.f;
  WeightTable tb{0u, 0u};
  // bf16: the weight of a logit of the current row from the row's table of
  // weight() (common.hpp); outside the table's window, weight() itself
  auto wt = [&](float l) -> uint64_t {
    if constexpr (sizeof(T) == 2) {
      bool in;
      const uint64_t w = table_weight(s_tab, tb, __float_as_uint(l) >> 16, in);
      return in ? w : weight(l, m, wc);
    } else {
      return weight(l, m, wc);
    }
  };
  while (true) {
    const int cur = s_cur;
    const T* row = logits + (base + cur) * static_cast<long>(V);
    const bool vec = aligned16(row) && (V % E == 0);
    // the row maximum (float maximum; -0 read as +0, as in the vocab pass)
    float vmax = -__builtin_huge_valf();
    if (vec) {
      // whole 16-byte vectors (V is a multiple of E): kLazyU loads in flight
      // per thread, then their maxima
      for (int p0 = 0; p0 < npass; p0 += kLazyU) {
        u32x4_t raw[kLazyU];
#pragma unroll
        for (int u = 0; u < kLazyU; ++u) {
          const long i = static_cast<long>(p0 + u) * kPass + static_cast<long>(tid) * E;
          raw[u] = p0 + u < npass && i < V ? *reinterpret_cast<const u32x4_t*>(row + i)
                                           : lazy_neg_inf<T>();
        }
#pragma unroll
        for (int u = 0; u < kLazyU; ++u) {
          float v[E];
          lazy_unpack<T>(raw[u], v);
#pragma unroll
          for (int e = 0; e < E; ++e) vmax = max(vmax, v[e]);
        }
      }
    } else {
      for (int p = 0; p < npass; ++p) {
        float v[E];
        lazy_load16<T>(row, static_cast<long>(p) * kPass + static_cast<long>(tid) * E, V, vec, v);
#pragma unroll
        for (int e = 0; e < E; ++e) vmax = max(vmax, v[e]);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) vmax = max(vmax, shfl_xor_f32(vmax, o));
    if (lane == 0) s_f[wave] = vmax;
    __syncthreads();
    m = s_f[0];
#pragma unroll
    for (int w = 1; w < kSampleWaves; ++w) m = max(m, s_f[w]);
    m = m + 0.0f;
    if constexpr (sizeof(T) == 2) {
      __syncthreads();   // the previous row's table is no longer read
      tb = fill_weight_table(s_tab, m, wc, tid, kSampleThreads);
      __syncthreads();
    }
    // the weights, summed per block of DDTREE_R_BLOCK tokens
    uint64_t bsum = 0;
    // one block of passes at a time (kPassPerBlock vectors per thread), its
    // loads issued together when the row is whole vectors
    for (int p0 = 0; p0 < npass; p0 += kPassPerBlock) {
      float v[kPassPerBlock][E];
      if (vec) {
        u32x4_t raw[kPassPerBlock];
#pragma unroll
        for (int u = 0; u < kPassPerBlock; ++u) {
          const long i = static_cast<long>(p0 + u) * kPass + static_cast<long>(tid) * E;
          raw[u] = p0 + u < npass && i < V ? *reinterpret_cast<const u32x4_t*>(row + i)
                                           : lazy_neg_inf<T>();
        }
#pragma unroll
        for (int u = 0; u < kPassPerBlock; ++u) lazy_unpack<T>(raw[u], v[u]);
      } else {
#pragma unroll
        for (int u = 0; u < kPassPerBlock; ++u)
          lazy_load16<T>(row, static_cast<long>(p0 + u) * kPass + static_cast<long>(tid) * E, V,
                         vec, v[u]);
      }
#pragma unroll
      for (int u = 0; u < kPassPerBlock; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          bsum += wt(v[u][e]);
          if (e & 1) __builtin_amdgcn_sched_barrier(0);
        }
      const uint64_t ws = wave_sum_u64(bsum);
      if (lane == 0) s_blkw[p0 / kPassPerBlock][wave] = ws;
      bsum = 0;
    }
    __syncthreads();
    if (tid < nb) {
      uint64_t bt = 0;
      for (int w = 0; w < kSampleWaves; ++w) bt += s_blkw[tid][w];
      s_Rb[tid] = bt;
    }
    __syncthreads();
    if (tid == 0) {
      uint64_t rres = 0;
      for (int k = 0; k < nb; ++k) rres += s_Rb[k];
      // the children in rank order: accept iff mulhi(u, R_res) < w(token)
      int nrej = 0, c = s_fc[cur];
      bool moved = false;
      while (c >= 0 && c < N && nrej < t.K) {
        const int tk = s_tok[c];
        const uint64_t wcur = (tk >= 0 && tk < V) ? wt(Elem<T>::get(row, tk)) : 0ull;
        if (__umul64hi(s_u0[c], rres) < wcur) {
          moved = true;
          break;
        }
        rres -= wcur;
        s_rej[nrej] = tk;
        ++nrej;
        c = s_ns[c];
      }
      const int a = s_a;
      if (moved && a < D) {
        outt[a] = s_tok[c];
        path[a + 1] = c;
        s_cur = c;
        s_a = a + 1;
        s_go = 1;
      } else {
        s_go = 0;
        s_nrej = nrej;
        s_rres = rres;
      }
    }
    __syncthreads();
    if (!s_go) break;
  }

  // residual draw over the stopping node's row: which weight block holds it
  // (the rejected tokens' weights come off their blocks), then 32 tokens per
  // thread within the block
  const int cur = s_cur, a = s_a, nrej = s_nrej;
  const T* row = logits + (base + cur) * static_cast<long>(V);
  if (wave == 0) {
    const uint64_t tdraw = __umul64hi(s_u1[cur], s_rres);
    uint64_t bs = 0;
    if (lane < nb) {
      bs = s_Rb[lane];
      for (int r = 0; r < nrej; ++r) {
        const int tk = s_rej[r];
        if (tk >= 0 && tk / DDTREE_R_BLOCK == lane) bs -= wt(Elem<T>::get(row, tk));
      }
    }
    const uint64_t incl = wave_incl_scan_u64(bs, lane);
    const uint64_t hit = __ballot(lane < nb && incl > tdraw);
    const int blk = hit ? __builtin_ctzll(hit) : nb - 1;
    const uint64_t ex = incl - bs;
    const uint32_t exl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex), blk));
    const uint32_t exh = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex >> 32), blk));
    if (lane == 0) {
      path[0] = 0;
      s_blk = blk;
      s_trem = tdraw - ((static_cast<uint64_t>(exh) << 32) | exl);
    }
    for (int k = a + 1 + lane; k <= D; k += kWave) {
      path[k] = -1;
      outt[k] = -1;
    }
  }
  __syncthreads();
  const uint64_t trem = s_trem;
  const long x0 = static_cast<long>(s_blk) * DDTREE_R_BLOCK + static_cast<long>(tid) * kTokPerThread;
  float v[32];
  load32<T>(row, x0, V, v);
  uint64_t sum = 0;
#pragma unroll
  for (int e = 0; e < 32; ++e) sum += wt(v[e]);
  for (int r = 0; r < nrej; ++r) {
    const long x = s_rej[r];
    if (x >= x0 && x < x0 + 32) sum -= wt(Elem<T>::get(row, x));
  }
  const uint64_t incl = wave_incl_scan_u64(sum, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int k = 0; k < wave; ++k) before += s_wave[k];
  const uint64_t excl = before + incl - sum;
  // the pick, by the wave holding the draw (as in sample_kernel)
  const uint64_t holder = __ballot(excl <= trem && trem < excl + sum);
  if (holder) {
    const int src = __builtin_ctzll(holder);
    const uint64_t excl_s = __shfl(excl, src, kWave);
    float x = -__builtin_huge_valf();
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const float tv = __shfl(v[e], src, kWave);
      x = lane == e ? tv : x;
    }
    const long xs = static_cast<long>(s_blk) * DDTREE_R_BLOCK +
                    static_cast<long>(wave * kWave + src) * kTokPerThread + lane;
    bool rej = false;
    for (int r = 0; r < nrej; ++r) rej |= (s_rej[r] == xs);
    const uint64_t w = lane < 32 && !rej ? wt(x) : 0ull;
    const uint64_t incl_s = wave_incl_scan_u64(w, lane);
    const uint64_t hit = __ballot(lane < 32 && excl_s + incl_s > trem);
    if (lane == 0) {
      const int pick = hit ? static_cast<int>(xs) + __builtin_ctzll(hit) : -1;
      outt[a] = pick;
      bonus[b] = pick;
    }
    release_system();   // as in sample_kernel
  }
  // accept_len last (as in sample_kernel)
  __syncthreads();
  if (tid == 0) {
    release_system();
    accept_len[b] = a;
  }
}


// ------------------------------------------------------------------ linear speculative sampling
// A chain of D drafted tokens, each drawn by the draft from its own softmax
// ("Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 3, linear
// DFlash at temperature T): position k accepts its token x with probability
// min(1, q(x) / p(x)), else draws from the residual max(0, q - p) and stops;
// after D acceptances the bonus comes from the target row D.  q and p are the
// exact integer laws w / R of the vocabulary pass (each row with its own
// maximum), so the accept test and the residual are integer arithmetic:
//   accept  iff  floor(u0 * wp(x) * Rq / 2^64) < wq(x) * Rp        (<= 147-bit)
//   r(y) = max(0, wq(y) Rp - wp(y) Rq) (< 2^83), Rr = sum r (< 2^101),
//   t = floor(u1 * Rr / 2^64), token = smallest y with running sum > t;
// if Rr = 0 the draw is from q.  One 1024-thread workgroup per request:
// thread 0 runs the accept tests; a residual is summed by the workgroup in
// passes of 8192 tokens (8 consecutive per thread), the pass holding t is
// found from the pass sums, and that pass is rescanned.
typedef unsigned __int128 u128;

__device__ __forceinline__ u128 mulhi_64x128(uint64_t u, u128 a) {
  const uint64_t lo = static_cast<uint64_t>(a), hi = static_cast<uint64_t>(a >> 64);
  return static_cast<u128>(__umul64hi(u, lo)) + static_cast<u128>(u) * hi;
}

__device__ __forceinline__ u128 shfl_xor_u128(u128 v, int m) {
  const uint64_t lo = __shfl_xor(static_cast<uint64_t>(v), m, kWave);
  const uint64_t hi = __shfl_xor(static_cast<uint64_t>(v >> 64), m, kWave);
  return (static_cast<u128>(hi) << 64) | lo;
}

__device__ __forceinline__ u128 shfl_up_u128(u128 v, int d) {
  const uint64_t lo = __shfl_up(static_cast<uint64_t>(v), d, kWave);
  const uint64_t hi = __shfl_up(static_cast<uint64_t>(v >> 64), d, kWave);
  return (static_cast<u128>(hi) << 64) | lo;
}

constexpr int kLinPass = kSampleThreads * 8;      // tokens per residual pass
constexpr int kLinMaxPass = 64 * DDTREE_R_BLOCK / kLinPass;

// 8 consecutive logits of a row as floats (one 16-byte load when `vec` and
// the 8 lie inside the row); past V read as -inf
template <typename T>
__device__ __forceinline__ void lin_load8(const T* row, long y0, int V, bool vec, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    if (vec && y0 + 8 <= V) {
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + y0);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = __uint_as_float((e & 1) ? (w[e >> 1] & 0xFFFF0000u) : (w[e >> 1] << 16));
      return;
    }
  } else {
    if (vec && y0 + 8 <= V) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(row + y0 + 4 * h);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * h + e] = __uint_as_float(w[e]);
      }
      return;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = y0 + e < V ? Elem<T>::get(row, y0 + e) : -__builtin_huge_valf();
}

// inclusive scan of a u128 over the workgroup in token (= thread) order;
// returns the exclusive prefix of this thread and writes the total
__device__ __forceinline__ u128 block_excl_scan_u128(u128 v, int lane, int wave, u128* s_w,
                                                     u128* total) {
  u128 incl = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const u128 o = shfl_up_u128(incl, d);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  u128 before = 0, tot = 0;
  for (int k = 0; k < kSampleWaves; ++k) {
    if (k < wave) before += s_w[k];
    tot += s_w[k];
  }
  __syncthreads();
  *total = tot;
  return before + incl - v;
}

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void linear_sample_kernel(
    const T* __restrict__ tlog, const T* __restrict__ dlog, int D, int V,
    const int32_t* __restrict__ dtok, const float* __restrict__ maxq,
    const uint64_t* __restrict__ Rq, const uint64_t* __restrict__ Rqb,
    const float* __restrict__ maxp, const uint64_t* __restrict__ Rp, WeightConsts wc,
    const uint64_t* __restrict__ uniforms, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ bonus) {
  constexpr bool kTab = sizeof(T) == 2;   // bf16: weights from LDS tables
  __shared__ u128 s_w[kSampleWaves];
  __shared__ u128 s_pass[kLinMaxPass];
  __shared__ u128 s_pw[kLinMaxPass][kSampleWaves];
  __shared__ uint64_t s_tq[kTab ? kTabEntries : 1], s_tp[kTab ? kTabEntries : 1];
  __shared__ uint64_t s_wave[kSampleWaves];
  __shared__ int s_k, s_mode, s_pick, s_blk;
  __shared__ u128 s_t;
  __shared__ uint64_t s_trem;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;
  int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);

  if (tid == 0) {
    // accept tests, position by position
    int k = 0;
    for (; k < D; ++k) {
      const long rq = static_cast<long>(b) * (D + 1) + k, rp = static_cast<long>(b) * D + k;
      const int x = dtok[rp];
      uint64_t wq = 0, wp = 0;
      if (x >= 0 && x < V) {
        wq = weight(Elem<T>::get(tlog + rq * V, x), maxq[rq], wc);
        wp = weight(Elem<T>::get(dlog + rp * V, x), maxp[rp], wc);
      }
      const u128 A = static_cast<u128>(wp) * Rq[rq], B = static_cast<u128>(wq) * Rp[rp];
      if (!(mulhi_64x128(uniforms[rq * 2 + 0], A) < B)) break;
      outt[k] = x;
    }
    s_k = k;
    // mode 0: draw from q of row k (the bonus, or a vanished residual); 1: residual
    s_mode = k < D ? 1 : 0;
    s_pick = -1;
  }
  __syncthreads();
  const int k = s_k;
  const long rq = static_cast<long>(b) * (D + 1) + k;
  const T* qrow = tlog + rq * V;
  const uint64_t u1 = uniforms[rq * 2 + 1];
  const float mq = maxq[rq];
  // bf16: the weights of target row k (and, for a residual, of draft row k)
  // from tables of weight() in LDS (common.hpp); outside a table's window,
  // weight() itself
  WeightTable tq{0u, 0u}, tp{0u, 0u};
  const int mode = s_mode;
  const long rp = static_cast<long>(b) * D + k;
  const float mp = mode == 1 ? maxp[rp] : 0.f;
  if constexpr (kTab) {
    tq = fill_weight_table(s_tq, mq, wc, tid, kSampleThreads);
    if (mode == 1) tp = fill_weight_table(s_tp, mp, wc, tid, kSampleThreads);
    __syncthreads();
  }
  auto wq_of = [&](float l) -> uint64_t {
    if constexpr (kTab) {
      bool in;
      const uint64_t w = table_weight(s_tq, tq, __float_as_uint(l) >> 16, in);
      return in ? w : weight(l, mq, wc);
    } else {
      return weight(l, mq, wc);
    }
  };
  auto wp_of = [&](float l) -> uint64_t {
    if constexpr (kTab) {
      bool in;
      const uint64_t w = table_weight(s_tp, tp, __float_as_uint(l) >> 16, in);
      return in ? w : weight(l, mp, wc);
    } else {
      return weight(l, mp, wc);
    }
  };
  if (mode == 1) {
    const T* prow = dlog + rp * V;
    const uint64_t Rqk = Rq[rq], Rpk = Rp[rp];
    const int npass = (V + kLinPass - 1) / kLinPass;
    const bool vq = aligned16(qrow) && V % 8 == 0, vp = aligned16(prow) && V % 8 == 0;
    // residual weight of one token from its two logits (0 past V: both -inf)
    auto rw = [&](float lq, float lp) -> u128 {
      const u128 a2 = static_cast<u128>(wq_of(lq)) * Rpk, b2 = static_cast<u128>(wp_of(lp)) * Rqk;
      return a2 > b2 ? a2 - b2 : 0;
    };
    // pass sums of the residual: each wave's share of a pass goes to LDS, one
    // barrier after the last pass
    for (int p = 0; p < npass; ++p) {
      const long y0 = static_cast<long>(p) * kLinPass + static_cast<long>(tid) * 8;
      float lq[8], lp[8];
      lin_load8<T>(qrow, y0, V, vq, lq);
      lin_load8<T>(prow, y0, V, vp, lp);
      u128 s = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) s += rw(lq[e], lp[e]);
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) s += shfl_xor_u128(s, m);
      if (lane == 0) s_pw[p][wave] = s;
    }
    __syncthreads();
    if (tid < npass) {
      u128 t = 0;
      for (int w = 0; w < kSampleWaves; ++w) t += s_pw[tid][w];
      s_pass[tid] = t;
    }
    __syncthreads();
    if (tid == 0) {
      u128 Rr = 0;
      for (int p = 0; p < npass; ++p) Rr += s_pass[p];
      if (Rr == 0) {
        s_mode = 0;   // q and p proportional: draw from q
      } else {
        const u128 t = mulhi_64x128(u1, Rr);
        u128 acc = 0;
        int p = 0;
        while (p < npass - 1 && acc + s_pass[p] <= t) acc += s_pass[p++];
        s_blk = p;
        s_t = t - acc;
      }
    }
    __syncthreads();
    if (s_mode == 1) {
      // rescan the pass holding the draw, in token order
      const u128 t = s_t;
      const long y0 = static_cast<long>(s_blk) * kLinPass + static_cast<long>(tid) * 8;
      float lq[8], lp[8];
      lin_load8<T>(qrow, y0, V, vq, lq);
      lin_load8<T>(prow, y0, V, vp, lp);
      u128 r[8], s = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r[e] = rw(lq[e], lp[e]);
        s += r[e];
      }
      u128 tot;
      const u128 excl = block_excl_scan_u128(s, lane, wave, s_w, &tot);
      if (s > 0 && excl <= t && t < excl + s) {
        u128 acc = excl;
        int pick = -1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc += r[e];
          if (pick < 0 && acc > t) pick = static_cast<int>(y0) + e;
        }
        s_pick = pick;
      }
      __syncthreads();
    }
  }
  if (s_mode == 0) {
    // draw from q of row k with the block sums of the vocabulary pass
    if (wave == 0) {
      const uint64_t tdraw = __umul64hi(u1, Rq[rq]);
      const uint64_t bs = lane < nb ? Rqb[rq * nb + lane] : 0ull;
      const uint64_t incl = wave_incl_scan_u64(bs, lane);
      const uint64_t hit = __ballot(lane < nb && incl > tdraw);
      const int blk = hit ? __builtin_ctzll(hit) : nb - 1;
      const uint64_t ex = incl - bs;
      const uint32_t exl = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex), blk));
      const uint32_t exh = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<uint32_t>(ex >> 32), blk));
      if (lane == 0) {
        s_blk = blk;
        s_trem = tdraw - ((static_cast<uint64_t>(exh) << 32) | exl);
      }
    }
    __syncthreads();
    const uint64_t trem = s_trem;
    const long x0 = static_cast<long>(s_blk) * DDTREE_R_BLOCK + static_cast<long>(tid) * kTokPerThread;
    float v[32];
    load32<T>(qrow, x0, V, v);
    uint64_t sum = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) sum += wq_of(v[e]);
    const uint64_t incl = wave_incl_scan_u64(sum, lane);
    if (lane == kWave - 1) s_wave[wave] = incl;
    __syncthreads();
    uint64_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    const uint64_t excl = before + incl - sum;
    if (excl <= trem && trem < excl + sum) {
      uint64_t acc = excl;
      int pick = -1;
      for (int e = 0; e < 32 && pick < 0; ++e) {
        acc += wq_of(v[e]);
        if (acc > trem) pick = static_cast<int>(x0) + e;
      }
      s_pick = pick;
    }
    __syncthreads();
  }
  if (tid == 0) {
    outt[k] = s_pick;
    bonus[b] = s_pick;
    for (int j = k + 1; j <= D; ++j) outt[j] = -1;
    // accept_len last, after a system-scope release (as in the tree walks)
    release_system();
    accept_len[b] = k;
  }
}

}  // namespace
}  // namespace ddt

extern "C" ddtree_status ddtree_verify_greedy(const ddtree_tree* tree, const int32_t* argmax,
                                              int32_t* accept_len, int32_t* path_nodes,
                                              int32_t* out_tokens, int32_t* bonus,
                                              hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_verify_greedy");
  if (st != DDTREE_OK) return st;
  if (!argmax || !accept_len || !path_nodes || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "ddtree_verify_greedy: null pointer");
  hipLaunchKernelGGL(greedy_kernel, dim3(tree->B), dim3(kWave), 0, stream, *tree, argmax,
                     accept_len, path_nodes, out_tokens, bonus);
  return check_launch("ddtree_verify_greedy");
}

extern "C" ddtree_status ddtree_verify_sample(const ddtree_tree* tree, const void* logits,
                                              ddtree_dtype dtype, int32_t V, const float* maxv,
                                              const uint64_t* R, const uint64_t* R_blocks,
                                              float temperature, const uint64_t* uniforms,
                                              int32_t* accept_len,
                                              int32_t* path_nodes, int32_t* out_tokens,
                                              int32_t* bonus, hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_verify_sample");
  if (st != DDTREE_OK) return st;
  if (!logits || !maxv || !R || !R_blocks || !uniforms || !accept_len || !path_nodes ||
      !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: null pointer");
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: temperature must be > 0 and finite");
  if (V < 1) return fail(DDTREE_EINVAL, "ddtree_verify_sample: V must be >= 1");
  if (V > kWave * DDTREE_R_BLOCK)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_verify_sample: V = %d exceeds %d", V,
                kWave * DDTREE_R_BLOCK);
  const WeightConsts wc = weight_consts(temperature);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL((sample_kernel<uint16_t, false>), dim3(tree->B), dim3(kSampleThreads), 0,
                       stream, *tree, static_cast<const uint16_t*>(logits), V, maxv, R, R_blocks,
                       wc, uniforms, accept_len, path_nodes, out_tokens, bonus, nullptr, nullptr);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL((sample_kernel<float, false>), dim3(tree->B), dim3(kSampleThreads), 0,
                       stream, *tree, static_cast<const float*>(logits), V, maxv, R, R_blocks, wc,
                       uniforms, accept_len, path_nodes, out_tokens, bonus, nullptr, nullptr);
  } else {
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: unknown dtype %d", static_cast<int>(dtype));
  }
  return check_launch("ddtree_verify_sample");
}

extern "C" ddtree_status ddtree_verify_sample_top_p(
    const ddtree_tree* tree, const void* logits, ddtree_dtype dtype, int32_t V, const float* maxv,
    const uint64_t* Rp, const uint64_t* Rp_blocks, const uint64_t* thr_w, const int32_t* thr_id,
    float temperature, const uint64_t* uniforms, int32_t* accept_len, int32_t* path_nodes,
    int32_t* out_tokens, int32_t* bonus, hipStream_t stream) {
  using namespace ddt;
  const char* who = "ddtree_verify_sample_top_p";
  ddtree_status st = check_tree(tree, who);
  if (st != DDTREE_OK) return st;
  if (!logits || !maxv || !Rp || !Rp_blocks || !thr_w || !thr_id || !uniforms || !accept_len ||
      !path_nodes || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "%s: null pointer", who);
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "%s: temperature must be > 0 and finite", who);
  if (V < 1) return fail(DDTREE_EINVAL, "%s: V must be >= 1", who);
  if (V > kWave * DDTREE_R_BLOCK)
    return fail(DDTREE_EUNSUPPORTED, "%s: V = %d exceeds %d", who, V, kWave * DDTREE_R_BLOCK);
  const WeightConsts wc = weight_consts(temperature);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL((sample_kernel<uint16_t, true>), dim3(tree->B), dim3(kSampleThreads), 0,
                       stream, *tree, static_cast<const uint16_t*>(logits), V, maxv, Rp,
                       Rp_blocks, wc, uniforms, accept_len, path_nodes, out_tokens, bonus, thr_w,
                       thr_id);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL((sample_kernel<float, true>), dim3(tree->B), dim3(kSampleThreads), 0,
                       stream, *tree, static_cast<const float*>(logits), V, maxv, Rp, Rp_blocks,
                       wc, uniforms, accept_len, path_nodes, out_tokens, bonus, thr_w, thr_id);
  } else {
    return fail(DDTREE_EINVAL, "%s: unknown dtype %d", who, static_cast<int>(dtype));
  }
  return check_launch(who);
}

extern "C" ddtree_status ddtree_verify_sample_lazy(const ddtree_tree* tree, const void* logits,
                                                   ddtree_dtype dtype, int32_t V,
                                                   float temperature, const uint64_t* uniforms,
                                                   int32_t* accept_len, int32_t* path_nodes,
                                                   int32_t* out_tokens, int32_t* bonus,
                                                   hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_verify_sample_lazy");
  if (st != DDTREE_OK) return st;
  if (!logits || !uniforms || !accept_len || !path_nodes || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "ddtree_verify_sample_lazy: null pointer");
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_verify_sample_lazy: temperature must be > 0 and finite");
  if (V < 1) return fail(DDTREE_EINVAL, "ddtree_verify_sample_lazy: V must be >= 1");
  if (V > kLazyMaxBlocks * DDTREE_R_BLOCK)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_verify_sample_lazy: V = %d exceeds %d", V,
                kLazyMaxBlocks * DDTREE_R_BLOCK);
  const WeightConsts wc = weight_consts(temperature);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL(sample_lazy_kernel<uint16_t>, dim3(tree->B), dim3(kSampleThreads), 0,
                       stream, *tree, static_cast<const uint16_t*>(logits), V, wc, uniforms,
                       accept_len, path_nodes, out_tokens, bonus);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL(sample_lazy_kernel<float>, dim3(tree->B), dim3(kSampleThreads), 0, stream,
                       *tree, static_cast<const float*>(logits), V, wc, uniforms, accept_len,
                       path_nodes, out_tokens, bonus);
  } else {
    return fail(DDTREE_EINVAL, "ddtree_verify_sample_lazy: unknown dtype %d",
                static_cast<int>(dtype));
  }
  return check_launch("ddtree_verify_sample_lazy");
}

extern "C" ddtree_status ddtree_verify_linear_sample(
    const void* target_logits, const void* draft_logits, ddtree_dtype dtype, int32_t B, int32_t D,
    int32_t V, const int32_t* draft_tokens, const float* maxq, const uint64_t* Rq,
    const uint64_t* Rq_blocks, const float* maxp, const uint64_t* Rp, float temperature,
    const uint64_t* uniforms, int32_t* accept_len, int32_t* out_tokens, int32_t* bonus,
    hipStream_t stream) {
  using namespace ddt;
  if (!target_logits || !draft_logits || !draft_tokens || !maxq || !Rq || !Rq_blocks || !maxp ||
      !Rp || !uniforms || !accept_len || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "ddtree_verify_linear_sample: null pointer");
  if (B < 1 || D < 1 || D > DDTREE_MAX_DEPTH || V < 1)
    return fail(DDTREE_EINVAL, "ddtree_verify_linear_sample: sizes out of range (B=%d D=%d V=%d)",
                B, D, V);
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_verify_linear_sample: temperature must be > 0 and finite");
  if (V > kWave * DDTREE_R_BLOCK)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_verify_linear_sample: V = %d exceeds %d", V,
                kWave * DDTREE_R_BLOCK);
  const WeightConsts wc = weight_consts(temperature);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL(linear_sample_kernel<uint16_t>, dim3(B), dim3(kSampleThreads), 0, stream,
                       static_cast<const uint16_t*>(target_logits),
                       static_cast<const uint16_t*>(draft_logits), D, V, draft_tokens, maxq, Rq,
                       Rq_blocks, maxp, Rp, wc, uniforms, accept_len, out_tokens, bonus);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL(linear_sample_kernel<float>, dim3(B), dim3(kSampleThreads), 0, stream,
                       static_cast<const float*>(target_logits),
                       static_cast<const float*>(draft_logits), D, V, draft_tokens, maxq, Rq,
                       Rq_blocks, maxp, Rp, wc, uniforms, accept_len, out_tokens, bonus);
  } else {
    return fail(DDTREE_EINVAL, "ddtree_verify_linear_sample: unknown dtype %d",
                static_cast<int>(dtype));
  }
  return check_launch("ddtree_verify_linear_sample");
}
