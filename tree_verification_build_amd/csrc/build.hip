// ddtree_build: best-first token tree, one wavefront per request.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's
// Tree-Parallel Evaluation Strategy", Section 1 steps 2-3: keep a frontier
// ordered by cumulative draft log-prob; take the best entry as the next node,
// then offer its best child and its next sibling; stop after `budget` nodes.
// The tree's visibility rows are ancestor-or-self sets; positions are
// prefix_len + depth ("The Tree That Couldn't Branch", "Hypothesis 3").
//
// Design: the frontier never holds more than budget + 1 <= 128 entries, so it
// lives in registers, two 64-bit keys per lane.  A key orders entries exactly
// as required (score desc, parent asc, rank asc) and carries the entry:
//   [63:32] order-preserving bits of the fp32 score
//   [31:24] 255 - parent   [23:16] 255 - rank   [15:8] depth   [7:0] pusher
// ("pusher" is the node whose taking offered this entry: the parent for a
// rank-0 child, the rank-1 sibling otherwise), so the best entry is one
// wave-wide 64-bit max.  A taken slot is refilled by the new child (or the
// new sibling); only when both exist does the sibling take a fresh slot.
// Node records accumulate in LDS and are written out coalesced at the end.
#include "common.hpp"

namespace ddt {
namespace {

constexpr int kMaxN = DDTREE_MAX_NODES;

__device__ __forceinline__ uint64_t make_key(float score, int parent, int rank, int depth,
                                             int pusher) {
  uint32_t lo = (static_cast<uint32_t>(255 - parent) << 24) |
                (static_cast<uint32_t>(255 - rank) << 16) |
                (static_cast<uint32_t>(depth) << 8) | static_cast<uint32_t>(pusher);
  return (static_cast<uint64_t>(ord_f32(score)) << 32) | lo;
}

__global__ __launch_bounds__(64) void build_kernel(const float* __restrict__ draft_lp,
                                                   const int32_t* __restrict__ draft_tok,
                                                   const int32_t* __restrict__ root_tok,
                                                   const int32_t* __restrict__ prefix_len,
                                                   int D, int K, int budget, ddtree_tree t) {
  extern __shared__ unsigned char smem[];
  float* s_lp = reinterpret_cast<float*>(smem);                    // [D*K]
  int32_t* s_tok = reinterpret_cast<int32_t*>(s_lp + D * K);      // [D*K]
  __shared__ float s_score[kMaxN];
  __shared__ int32_t s_token[kMaxN], s_parent[kMaxN], s_depth[kMaxN], s_rank[kMaxN];
  __shared__ int32_t s_fc[kMaxN], s_ns[kMaxN];
  __shared__ uint64_t s_vis[kMaxN][2];

  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = budget + 1;
  const int DK = D * K;
  for (int i = lane; i < DK; i += kWave) {
    s_lp[i] = draft_lp[static_cast<long>(b) * DK + i];
    s_tok[i] = draft_tok[static_cast<long>(b) * DK + i];
  }
  for (int i = lane; i < kMaxN; i += kWave) {
    s_fc[i] = -1;
    s_ns[i] = -1;
  }
  if (lane == 0) {
    s_score[0] = 0.0f;
    s_token[0] = root_tok[b];
    s_parent[0] = -1;
    s_depth[0] = 0;
    s_rank[0] = -1;
    s_vis[0][0] = 1ull;
    s_vis[0][1] = 0ull;
  }
  __syncthreads();

  uint64_t key0 = 0, key1 = 0;  // slots lane and lane + 64
  int nslots = 1;
  if (lane == 0) key0 = make_key(0.0f + s_lp[0], 0, 0, 1, 0);
  int count = 1;
  while (count < N) {
    uint64_t best = wave_max_u64(key0 > key1 ? key0 : key1);
    if (best == 0) break;  // frontier empty
    const uint32_t lo = static_cast<uint32_t>(best);
    const float score = unord_f32(static_cast<uint32_t>(best >> 32));
    const int parent = 255 - static_cast<int>(lo >> 24);
    const int rank = 255 - static_cast<int>((lo >> 16) & 0xFF);
    const int depth = static_cast<int>((lo >> 8) & 0xFF);
    const int pusher = static_cast<int>(lo & 0xFF);
    const int i = count++;

    uint64_t child = 0, sib = 0;
    if (depth < D) child = make_key(score + s_lp[depth * K], i, 0, depth + 1, i);
    if (rank + 1 < K)
      sib = make_key(s_score[parent] + s_lp[(depth - 1) * K + rank + 1], parent, rank + 1, depth, i);
    const uint64_t refill = child ? child : sib;
    if (key0 == best) key0 = refill;
    if (key1 == best) key1 = refill;
    if (child && sib) {
      if (lane == (nslots & 63)) {
        if (nslots < 64) key0 = sib; else key1 = sib;
      }
      ++nslots;
    }
    if (lane == 0) {
      s_score[i] = score;
      s_token[i] = s_tok[(depth - 1) * K + rank];
      s_parent[i] = parent;
      s_depth[i] = depth;
      s_rank[i] = rank;
      uint64_t v0 = s_vis[parent][0], v1 = s_vis[parent][1];
      if (i < 64) v0 |= 1ull << i; else v1 |= 1ull << (i - 64);
      s_vis[i][0] = v0;
      s_vis[i][1] = v1;
      if (rank == 0) s_fc[parent] = i; else s_ns[pusher] = i;
    }
  }
  __syncthreads();

  const long base = static_cast<long>(b) * N;
  const int W = t.W;
  for (int i = lane; i < N; i += kWave) {
    const bool ok = i < count;
    t.token[base + i] = ok ? s_token[i] : -1;
    t.parent[base + i] = ok ? s_parent[i] : -1;
    t.depth[base + i] = ok ? s_depth[i] : -1;
    t.rank[base + i] = ok ? s_rank[i] : -1;
    t.position[base + i] = ok ? prefix_len[b] + s_depth[i] : -1;
    t.first_child[base + i] = ok ? s_fc[i] : -1;
    t.next_sibling[base + i] = ok ? s_ns[i] : -1;
    t.score[base + i] = ok ? s_score[i] : -__builtin_huge_valf();
    for (int w = 0; w < W; ++w) t.vis[(base + i) * W + w] = ok ? s_vis[i][w] : 0ull;
  }
  if (lane == 0) t.num_nodes[b] = count;
}

}  // namespace

ddtree_status check_tree(const ddtree_tree* t, const char* who) {
  if (!t) return fail(DDTREE_EINVAL, "%s: tree is null", who);
  if (!t->token || !t->parent || !t->depth || !t->rank || !t->position || !t->first_child ||
      !t->next_sibling || !t->score || !t->vis || !t->num_nodes)
    return fail(DDTREE_EINVAL, "%s: a tree array is null", who);
  if (t->B < 1 || t->N < 2 || t->N > DDTREE_MAX_NODES || t->W != (t->N + 63) / 64 ||
      t->D < 1 || t->D > DDTREE_MAX_DEPTH || t->K < 1 || t->K > DDTREE_MAX_TOPK)
    return fail(DDTREE_EINVAL, "%s: tree sizes out of range (B=%d N=%d D=%d K=%d W=%d)", who,
                t->B, t->N, t->D, t->K, t->W);
  return DDTREE_OK;
}

}  // namespace ddt

extern "C" ddtree_status ddtree_build(const float* draft_lp, const int32_t* draft_tok,
                                      const int32_t* root_tok, const int32_t* prefix_len,
                                      int32_t B, int32_t D, int32_t K, int32_t budget,
                                      const ddtree_tree* tree, hipStream_t stream) {
  using namespace ddt;
  if (!draft_lp || !draft_tok || !root_tok || !prefix_len)
    return fail(DDTREE_EINVAL, "ddtree_build: null input pointer");
  ddtree_status st = check_tree(tree, "ddtree_build");
  if (st != DDTREE_OK) return st;
  if (budget < 1 || budget + 1 > DDTREE_MAX_NODES)
    return fail(DDTREE_EINVAL, "ddtree_build: budget %d out of [1, %d]", budget,
                DDTREE_MAX_NODES - 1);
  if (tree->N != budget + 1 || tree->B != B || tree->D != D || tree->K != K)
    return fail(DDTREE_EINVAL, "ddtree_build: tree sizes do not match B/D/K/budget");
  const size_t smem = static_cast<size_t>(D) * K * (sizeof(float) + sizeof(int32_t));
  hipLaunchKernelGGL(build_kernel, dim3(B), dim3(kWave), smem, stream, draft_lp, draft_tok,
                     root_tok, prefix_len, D, K, budget, *tree);
  return check_launch("ddtree_build");
}
