// ddtree_build: best-first token tree, one wavefront per request.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's
// Tree-Parallel Evaluation Strategy", Section 1 steps 2-3: keep a frontier
// ordered by cumulative draft log-prob; take the best entry as the next node,
// then offer its best child and its next sibling; stop after `budget` nodes.
// The tree's visibility rows are ancestor-or-self sets; positions are
// prefix_len + depth ("The Tree That Couldn't Branch", "Hypothesis 3").
//
// Design: one wavefront per request.  Every taken node p has at most one
// pending offer, its next child not yet taken (the rank-0 child when p is
// taken, then each next sibling as the previous one is taken), so the
// frontier is a set of slots, slot p in lane p % 64 (two register pairs for
// N > 64), each holding a 64-bit key that orders entries exactly as required
// (score desc, parent asc, rank asc) and carries the entry:
//   [63:32] order-preserving bits of the fp32 score
//   [31:24] 255 - parent   [23:16] 255 - rank   [15:8] depth   [7:0] pusher
// ("pusher" is the node whose taking offered this entry: the parent for a
// rank-0 child, the previous sibling otherwise).  A step takes the slot with
// the largest key (a DPP maximum of the high words; the low words only break
// score ties), records it as node i, and writes two keys: node i's best child
// into slot i and the parent's next child into slot parent (0 for "none").
// The step is a serial chain of ~85 instructions in one wave, so the loop
// does nothing else: tokens, positions, child / sibling links and visibility
// rows are rebuilt afterwards, all lanes in parallel (visibility by pointer
// jumping over parent links).  The draft top-k table (D*K <= 256 entries) is
// spread over the lanes and read with v_readlane.
#include "common.hpp"

namespace ddt {
namespace {

__device__ __forceinline__ uint64_t make_key_bits(uint32_t ord_score, int parent, int rank,
                                                  int depth, int pusher) {
  const uint32_t lo = (static_cast<uint32_t>(255 - parent) << 24) |
                      (static_cast<uint32_t>(255 - rank) << 16) |
                      (static_cast<uint32_t>(depth) << 8) | static_cast<uint32_t>(pusher);
  return (static_cast<uint64_t>(ord_score) << 32) | lo;
}

__device__ __forceinline__ uint64_t make_key(float score, int parent, int rank, int depth,
                                             int pusher) {
  return make_key_bits(ord_f32(score), parent, rank, depth, pusher);
}

// fp32 bits of the value an order-preserving key word encodes
__device__ __forceinline__ uint32_t unord_f32_bits(uint32_t o) {
  return (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
}

// order-preserving bits of fp32 bits (-0 as +0), as plain integer operations
__device__ __forceinline__ uint32_t ord_bits(uint32_t u) {
  u = u == 0x80000000u ? 0u : u;
  const uint32_t m = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
  return u ^ (m | 0x80000000u);
}

// value of a per-lane register table at flat index idx (uniform): one readlane
// when the table fits one register (D*K <= 64), else a scalar select of four
template <int REGS>
__device__ __forceinline__ uint32_t table_at(const uint32_t (&r)[4], int idx) {
  if (REGS == 1) return __builtin_amdgcn_readlane(r[0], idx);
  const int w = idx >> 6, l = idx & 63;
  const uint32_t a0 = __builtin_amdgcn_readlane(r[0], l), a1 = __builtin_amdgcn_readlane(r[1], l);
  const uint32_t a2 = __builtin_amdgcn_readlane(r[2], l), a3 = __builtin_amdgcn_readlane(r[3], l);
  return w == 0 ? a0 : w == 1 ? a1 : w == 2 ? a2 : a3;
}

// Maximum over the wavefront with DPP: within each row of 16 lanes (quad_perm
// swaps, row_ror 4 and 8), then row_bcast15 / row_bcast31 carry the running
// maximum into the last row; lane 63 ends with the total.
__device__ __forceinline__ uint32_t wave_max_bcast_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x142, 0xA, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x143, 0xC, 0xF, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 63));
}

// lane-varying gather from the per-lane table (ds_bpermute)
template <int REGS>
__device__ __forceinline__ uint32_t table_gather(const uint32_t (&r)[4], int idx) {
  const int l = idx & 63, w = idx >> 6;
  uint32_t v = __shfl(r[0], l, 64);
  if (REGS > 1) {
    const uint32_t v1 = __shfl(r[1], l, 64), v2 = __shfl(r[2], l, 64), v3 = __shfl(r[3], l, 64);
    v = w == 1 ? v1 : w == 2 ? v2 : w == 3 ? v3 : v;
  }
  return v;
}

template <int REGS, bool TWO>
__global__ __launch_bounds__(64) void build_kernel(const float* __restrict__ draft_lp,
                                                   const int32_t* __restrict__ draft_tok,
                                                   const int32_t* __restrict__ root_tok,
                                                   const int32_t* __restrict__ prefix_len,
                                                   int D, int K, int budget, ddtree_tree t) {
  __shared__ int32_t s_fc[DDTREE_MAX_NODES], s_ns[DDTREE_MAX_NODES];
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int N = budget + 1;
  const int DK = D * K;
  // draft table: entry i = d * K + r in register i / 64 of lane i % 64
  uint32_t lp_r[4], tok_r[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int i = w * 64 + lane;
    lp_r[w] = (w < REGS && i < DK) ? __float_as_uint(draft_lp[static_cast<long>(b) * DK + i]) : 0u;
    tok_r[w] = (w < REGS && i < DK) ? static_cast<uint32_t>(draft_tok[static_cast<long>(b) * DK + i]) : 0u;
  }
  s_fc[lane] = -1;
  s_ns[lane] = -1;
  if (TWO) {
    s_fc[lane + 64] = -1;
    s_ns[lane + 64] = -1;
  }

  // records: the taken key of node i sits in lane i % 64 of (rh0, rl0) or (rh1, rl1);
  // the root's record carries score +0.0 (its other fields are never read)
  uint32_t rh0 = lane == 0 ? ord_f32(0.0f) : 0u, rl0 = 0u, rh1 = 0u, rl1 = 0u;
  // frontier slots: every taken node p has at most one pending offer, its
  // next child not yet taken, and that offer sits in slot p (lane p % 64 of
  // (sh0, sl0) or (sh1, sl1)); key 0 = none.  The root's first child starts
  // in slot 0.
  const uint64_t first = make_key(0.0f + __uint_as_float(table_at<REGS>(lp_r, 0)), 0, 0, 1, 0);
  uint32_t sh0 = lane == 0 ? static_cast<uint32_t>(first >> 32) : 0u;
  uint32_t sl0 = lane == 0 ? static_cast<uint32_t>(first) : 0u;
  uint32_t sh1 = 0u, sl1 = 0u;

  int count = 1;
  for (; count < N; ++count) {
    // the best slot: largest key; the high word (score) decides unless tied
    uint32_t mh = sh0, ml = sl0;
    if (TWO) {
      const bool in1 = ((static_cast<uint64_t>(sh1) << 32) | sl1) > ((static_cast<uint64_t>(sh0) << 32) | sl0);
      mh = in1 ? sh1 : sh0;
      ml = in1 ? sl1 : sl0;
    }
    const uint32_t bh = wave_max_bcast_u32(mh);
    if (bh == 0) break;  // no offers left
    const uint64_t tied = __ballot(mh == bh);
    int w = __builtin_ctzll(tied);
    if (tied & (tied - 1)) w = __builtin_ctzll(__ballot(mh == bh && ml == wave_max_bcast_u32(mh == bh ? ml : 0u)));
    // readlane yields a signed int: cast before widening, or the low word sign-extends
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(ml, w));
    const int parent = 255 - static_cast<int>(lo >> 24);
    const int rank = 255 - static_cast<int>((lo >> 16) & 0xFF);
    const int depth = static_cast<int>((lo >> 8) & 0xFF);
    const int i = count;
    const uint32_t pscore = unord_f32_bits(static_cast<uint32_t>(
        __builtin_amdgcn_readlane(TWO && parent >= 64 ? rh1 : rh0, parent & 63)));
    // record node i (branch-free: lane i of the low registers or lane i - 64
    // of the high ones)
    const bool at_i0 = lane == i, at_i1 = TWO && lane + 64 == i;
    const bool at_p0 = lane == parent, at_p1 = TWO && lane + 64 == parent;
    rh0 = at_i0 ? bh : rh0;
    rl0 = at_i0 ? lo : rl0;
    if (TWO) {
      rh1 = at_i1 ? bh : rh1;
      rl1 = at_i1 ? lo : rl1;
    }
    // offers: node i's best child goes to slot i, the parent's next child
    // replaces the taken one in slot parent (key 0 when there is none)
    const float lpc = __uint_as_float(table_at<REGS>(lp_r, min(depth, D - 1) * K));
    const float lps = __uint_as_float(table_at<REGS>(lp_r, (depth - 1) * K + min(rank + 1, K - 1)));
    const uint32_t cs = __float_as_uint(__uint_as_float(unord_f32_bits(bh)) + lpc);
    const uint32_t ss = __float_as_uint(__uint_as_float(pscore) + lps);
    const uint64_t kc = depth < D ? make_key_bits(ord_bits(cs), i, 0, depth + 1, i) : 0ull;
    const uint64_t ks = rank + 1 < K ? make_key_bits(ord_bits(ss), parent, rank + 1, depth, i) : 0ull;
    const uint32_t kch = static_cast<uint32_t>(kc >> 32), kcl = static_cast<uint32_t>(kc);
    const uint32_t ksh = static_cast<uint32_t>(ks >> 32), ksl = static_cast<uint32_t>(ks);
    sh0 = at_i0 ? kch : at_p0 ? ksh : sh0;
    sl0 = at_i0 ? kcl : at_p0 ? ksl : sl0;
    if (TWO) {
      sh1 = at_i1 ? kch : at_p1 ? ksh : sh1;
      sl1 = at_i1 ? kcl : at_p1 ? ksl : sl1;
    }
  }

  // rebuild the node arrays from the records, every lane in parallel
  const long base = static_cast<long>(b) * N;
  const int W = t.W;
  int par[2], dep[2], rnk[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = s * 64 + lane;
    const uint32_t lo = s == 0 ? rl0 : rl1;
    const bool ok = i < count && (s == 0 || TWO);
    par[s] = ok && i > 0 ? 255 - static_cast<int>(lo >> 24) : -1;
    rnk[s] = ok && i > 0 ? 255 - static_cast<int>((lo >> 16) & 0xFF) : -1;
    dep[s] = ok ? (i > 0 ? static_cast<int>((lo >> 8) & 0xFF) : 0) : -1;
    if (ok && i > 0) {
      const int pusher = static_cast<int>(lo & 0xFF);
      if (rnk[s] == 0) s_fc[par[s]] = i; else s_ns[pusher] = i;
    }
  }
  // visibility rows by pointer jumping: after round k each row holds the node's
  // 2^k nearest ancestors (and itself); depth <= 64 needs at most 7 rounds
  uint32_t va[2][4], anc[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = s * 64 + lane;
#pragma unroll
    for (int w = 0; w < 4; ++w) va[s][w] = 0u;
    if (dep[s] >= 0) {
      va[s][i >> 5] |= 1u << (i & 31);
      if (par[s] >= 0) va[s][par[s] >> 5] |= 1u << (par[s] & 31);
    }
    anc[s] = par[s] >= 0 ? static_cast<uint32_t>(par[s]) : 0xFFFFFFFFu;
  }
  for (int jump = 1; jump < D; jump <<= 1) {
    uint32_t nv[2][4], na[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t a = anc[s];
      const int src = static_cast<int>(a & 63);
      const bool hi = TWO && a != 0xFFFFFFFFu && a >= 64;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t g0 = __shfl(va[0][w], src, 64);
        const uint32_t g1 = TWO ? __shfl(va[1][w], src, 64) : 0u;
        nv[s][w] = va[s][w] | (a == 0xFFFFFFFFu ? 0u : (hi ? g1 : g0));
      }
      const uint32_t a0 = __shfl(anc[0], src, 64);
      const uint32_t a1 = TWO ? __shfl(anc[1], src, 64) : 0xFFFFFFFFu;
      na[s] = a == 0xFFFFFFFFu ? a : (hi ? a1 : a0);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      anc[s] = na[s];
#pragma unroll
      for (int w = 0; w < 4; ++w) va[s][w] = nv[s][w];
    }
  }
  // tokens: gathered with every lane active
  int tg[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    tg[s] = static_cast<int>(table_gather<REGS>(tok_r, max(0, (dep[s] - 1) * K + rnk[s])));
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int i = s * 64 + lane;
    if (i < N) {
      const bool ok = dep[s] >= 0;
      const uint32_t hi = s == 0 ? rh0 : rh1;
      t.token[base + i] = !ok ? -1 : i == 0 ? root_tok[b] : tg[s];
      t.parent[base + i] = par[s];
      t.depth[base + i] = dep[s];
      t.rank[base + i] = rnk[s];
      t.position[base + i] = ok ? prefix_len[b] + dep[s] : -1;
      t.first_child[base + i] = ok ? s_fc[i] : -1;
      t.next_sibling[base + i] = ok ? s_ns[i] : -1;
      t.score[base + i] = ok ? unord_f32(hi) : -__builtin_huge_valf();
      t.vis[(base + i) * W] = (static_cast<uint64_t>(va[s][1]) << 32) | va[s][0];
      if (W > 1) t.vis[(base + i) * W + 1] = (static_cast<uint64_t>(va[s][3]) << 32) | va[s][2];
    }
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
  if (D * K > 256)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_build: depth * top-k = %d exceeds 256", D * K);
  const bool small_table = D * K <= 64, one_list = budget + 1 <= 64;
  const dim3 g(B), blk(kWave);
  if (small_table && one_list)
    hipLaunchKernelGGL((build_kernel<1, false>), g, blk, 0, stream, draft_lp, draft_tok, root_tok,
                       prefix_len, D, K, budget, *tree);
  else if (small_table)
    hipLaunchKernelGGL((build_kernel<1, true>), g, blk, 0, stream, draft_lp, draft_tok, root_tok,
                       prefix_len, D, K, budget, *tree);
  else if (one_list)
    hipLaunchKernelGGL((build_kernel<4, false>), g, blk, 0, stream, draft_lp, draft_tok, root_tok,
                       prefix_len, D, K, budget, *tree);
  else
    hipLaunchKernelGGL((build_kernel<4, true>), g, blk, 0, stream, draft_lp, draft_tok, root_tok,
                       prefix_len, D, K, budget, *tree);
  return check_launch("ddtree_build");
}
