// ddtree_verify_greedy / ddtree_verify_sample: verified-tree walks.
//
// Greedy ("Dissecting DDTree's Tree-Parallel Evaluation Strategy", Section 1
// step 5): one wavefront per request.  Every lane holds two nodes; a step of
// the walk is one ballot over "parent == cur and token == argmax[cur]".
//
// Sampled (same page, Section 3; "Implementing Temperature-Aware Tree
// Sampling for DDTree", "Path B"): one 1024-thread workgroup per request.
// Wave 0 first gathers, in parallel, the weight every node's token has under
// its parent's target row, then walks the tree with exact integer draws
// (t = mulhi(u, R_res); accept iff t < w).  If the walk stops, the whole
// workgroup recomputes the weights of the stopping node's row, removes the
// rejected tokens, and finds the bonus token by an exact integer prefix scan.
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
  const int N = t.N, D = t.D;
  const long base = static_cast<long>(b) * N;
  // the tree and argmax rows are read before num_nodes is known (all N
  // entries exist), so that the loads do not wait for it
  int par[2], tok[2], am[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + s * kWave;
    par[s] = j < N ? t.parent[base + j] : -2;
    tok[s] = j < N ? t.token[base + j] : -2;
    am[s] = j < N ? argmax[base + j] : -1;
  }
  const int nn = t.num_nodes[b];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + s * kWave;
    const bool ok = j < nn;
    par[s] = ok ? par[s] : -2;
    tok[s] = ok ? tok[s] : -2;
    if (j < N) s_am[j] = ok ? am[s] : -1;
  }
  __syncthreads();
  int32_t* path = path_nodes + static_cast<long>(b) * (D + 1);
  int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
  int cur = 0, a = 0;
  while (a < D) {
    const int target = s_am[cur];
    const uint64_t m0 = __ballot(par[0] == cur && tok[0] == target);
    const uint64_t m1 = __ballot(par[1] == cur && tok[1] == target);
    if (!m0 && !m1) break;
    const int c = m0 ? __builtin_ctzll(m0) : kWave + __builtin_ctzll(m1);
    if (lane == 0) outt[a] = target;
    cur = c;
    ++a;
    if (lane == 0) path[a] = c;
  }
  const int bon = s_am[cur];
  for (int k = lane; k <= D; k += kWave) {
    if (k > a) {
      path[k] = -1;
      outt[k] = -1;
    }
  }
  if (lane == 0) {
    path[0] = 0;
    outt[a] = bon;
    accept_len[b] = a;
    bonus[b] = bon;
  }
}

constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;

template <typename T>
__global__ __launch_bounds__(kSampleThreads) void sample_kernel(
    ddtree_tree t, const T* __restrict__ logits, int V, const float* __restrict__ maxv,
    const uint64_t* __restrict__ R, WeightConsts wc, const uint64_t* __restrict__ uniforms,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ path_nodes,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ bonus) {
  __shared__ uint64_t s_w[kMaxN];
  __shared__ int32_t s_tok[kMaxN], s_fc[kMaxN], s_ns[kMaxN];
  __shared__ int32_t s_rej[DDTREE_MAX_TOPK];
  __shared__ uint64_t s_wave[kSampleWaves];
  __shared__ int s_nrej, s_cur, s_a;
  __shared__ uint64_t s_t, s_found_excl;
  __shared__ int s_found_thread;

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int N = t.N, D = t.D;
  const long base = static_cast<long>(b) * N;
  const int nn = t.num_nodes[b];

  if (wave == 0) {
    // weights of every node's token under its parent's row
    for (int j = lane; j < N; j += kWave) {
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
        }
      }
      s_w[j] = w;
      s_tok[j] = tk;
      s_fc[j] = fc;
      s_ns[j] = ns;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // the walk (every lane follows the same uniform path)
    int32_t* path = path_nodes + static_cast<long>(b) * (D + 1);
    int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
    int cur = 0, a = 0, nrej = 0;
    uint64_t rres = 0;
    // both loops are capped (depth <= D, children <= K), so a malformed tree cannot hang
    while (true) {
      rres = R[base + cur];
      nrej = 0;
      int c = s_fc[cur];
      bool moved = false;
      while (c >= 0 && c < N && nrej < t.K) {
        const uint64_t tt = __umul64hi(uniforms[(base + c) * 2 + 0], rres);
        const uint64_t wcur = s_w[c];
        if (tt < wcur) {
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
    if (lane == 0) {
      path[0] = 0;
      s_found_thread = -1;
      s_nrej = nrej;
      s_cur = cur;
      s_a = a;
      s_t = __umul64hi(uniforms[(base + cur) * 2 + 1], rres);
      accept_len[b] = a;
    }
    for (int k = a + 1 + lane; k <= D; k += kWave) {
      path[k] = -1;
      outt[k] = -1;
    }
  }
  __syncthreads();

  // residual draw over the stopping node's row
  const int cur = s_cur;
  const int nrej = s_nrej;
  const uint64_t tdraw = s_t;
  const float m = maxv[base + cur];
  const T* row = logits + (base + cur) * static_cast<long>(V);
  const int seg = (V + kSampleThreads - 1) / kSampleThreads;
  const int lo = min(V, tid * seg), hi = min(V, lo + seg);
  uint64_t sum = 0;
  for (int x = lo; x < hi; ++x) sum += weight(Elem<T>::get(row, x), m, wc);
  for (int r = 0; r < nrej; ++r) {
    const int x = s_rej[r];
    if (x >= lo && x < hi) sum -= weight(Elem<T>::get(row, x), m, wc);
  }
  // exclusive prefix of per-thread sums over the workgroup
  const uint64_t incl = wave_incl_scan_u64(sum, lane);
  if (lane == kWave - 1) s_wave[wave] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int w = 0; w < wave; ++w) before += s_wave[w];
  const uint64_t excl = before + incl - sum;
  if (excl <= tdraw && tdraw < excl + sum) {
    s_found_thread = tid;
    s_found_excl = excl;
  }
  __syncthreads();
  if (tid == s_found_thread) {
    uint64_t acc = s_found_excl;
    int pick = -1;
    for (int x = lo; x < hi; ++x) {
      bool rej = false;
      for (int r = 0; r < nrej; ++r) rej |= (s_rej[r] == x);
      if (rej) continue;
      acc += weight(Elem<T>::get(row, x), m, wc);
      if (acc > tdraw) {
        pick = x;
        break;
      }
    }
    int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
    outt[s_a] = pick;
    bonus[b] = pick;
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
                                              const uint64_t* R, float temperature,
                                              const uint64_t* uniforms, int32_t* accept_len,
                                              int32_t* path_nodes, int32_t* out_tokens,
                                              int32_t* bonus, hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_verify_sample");
  if (st != DDTREE_OK) return st;
  if (!logits || !maxv || !R || !uniforms || !accept_len || !path_nodes || !out_tokens || !bonus)
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: null pointer");
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: temperature must be > 0 and finite");
  if (V < 1) return fail(DDTREE_EINVAL, "ddtree_verify_sample: V must be >= 1");
  const WeightConsts wc = weight_consts(temperature);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL(sample_kernel<uint16_t>, dim3(tree->B), dim3(kSampleThreads), 0, stream,
                       *tree, static_cast<const uint16_t*>(logits), V, maxv, R, wc, uniforms,
                       accept_len, path_nodes, out_tokens, bonus);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL(sample_kernel<float>, dim3(tree->B), dim3(kSampleThreads), 0, stream,
                       *tree, static_cast<const float*>(logits), V, maxv, R, wc, uniforms,
                       accept_len, path_nodes, out_tokens, bonus);
  } else {
    return fail(DDTREE_EINVAL, "ddtree_verify_sample: unknown dtype %d", static_cast<int>(dtype));
  }
  return check_launch("ddtree_verify_sample");
}
