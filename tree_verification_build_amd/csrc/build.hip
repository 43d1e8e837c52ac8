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
// into slot i and the parent's next child into slot parent.  The scores of
// those two offers are computed beforehand by every lane for its own slot,
// alongside the maximum, so the step's dependent chain after the maximum is
// three lane reads and a few lane writes (~70 instructions per step in all).
// Offers that do not exist get key 0, below every real key (a real offer may
// score -inf), and are never taken: the loop runs exactly as many steps as
// the tree can hold nodes.  Tokens, positions, child / sibling links and visibility rows
// are rebuilt afterwards, all lanes in parallel (visibility by pointer
// jumping over parent links).
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

// Maximum over the wavefront with DPP: within each row of 16 lanes (quad_perm
// swaps, row_ror 4 and 8), then row_bcast15 / row_bcast31 carry the running
// maximum into the last row; lane 63 ends with the total.  HALF: only lanes
// 0-31 hold candidates, so row_bcast15 alone brings their maximum to lane 31.
template <bool HALF = false>
__device__ __forceinline__ uint32_t wave_max_bcast_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x142, 0xA, 0xF, false)));
  if constexpr (HALF) return static_cast<uint32_t>(__builtin_amdgcn_readlane(v, 31));
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

constexpr int kRow = 128;   // LDS row stride of the log-prob table (> DDTREE_MAX_TOPK)

}  // namespace
}  // namespace ddt

// v_writelane_b32 (write one lane of a VGPR from a scalar), reached through
// its LLVM intrinsic so that the compiler still handles its hazards
extern "C" __device__ int ddt_writelane_i32(int val, int lane, int old) __asm("llvm.amdgcn.writelane.i32");

namespace ddt {
namespace {

__device__ __forceinline__ uint32_t put_lane(uint32_t old, uint32_t val, int lane) {
  return static_cast<uint32_t>(ddt_writelane_i32(static_cast<int>(val), lane, static_cast<int>(old)));
}
__device__ __forceinline__ float put_lane(float old, float val, int lane) {
  return __builtin_bit_cast(float, ddt_writelane_i32(__builtin_bit_cast(int, val), lane,
                                                     __builtin_bit_cast(int, old)));
}

// TWO: node records in two register sets (N > 64); SLOTS2: the frontier's
// slots too (N > 65: with N = 65 the last pop writes slot 64, which no pop
// reads, so the frontier fits one set); HALF: N <= 33, so the slots a pop
// reads (0 .. N - 2) lie in lanes 0-31.
template <int REGS, bool TWO, bool SLOTS2, bool HALF>
__global__ __launch_bounds__(64) void build_kernel(const float* __restrict__ draft_lp,
                                                   const int32_t* __restrict__ draft_tok,
                                                   const int32_t* __restrict__ root_tok,
                                                   const int32_t* __restrict__ prefix_len,
                                                   int D, int K, int budget, ddtree_tree t) {
  __shared__ int32_t s_fc[DDTREE_MAX_NODES], s_ns[DDTREE_MAX_NODES];
  extern __shared__ float s_table[];   // (D + 2) * kRow floats
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

  // The log-prob table in LDS with a fixed row stride: row d - 1 holds depth
  // d, ranks 0..K-1, then -inf up to kRow; rows D and D + 1 (depths D + 1,
  // D + 2: children of depth-D nodes and their offers) are all -inf.
  // An offer that does not exist (a child below depth D, a sibling past rank
  // K - 1) reads -inf here; its key is then set below every real key.
  float* s_T = s_table;
#pragma unroll 1
  for (int e = lane; e < (D + 2) * kRow; e += 64) s_T[e] = -__builtin_huge_valf();
  __syncthreads();
#pragma unroll
  for (int w = 0; w < REGS; ++w) {
    const int e = w * 64 + lane;
    if (e < DK) s_T[(e / K) * kRow + e % K] = __uint_as_float(lp_r[w]);
  }
  __syncthreads();

  // Per lane, for set 0 (nodes / slots 0..63) and set 1 (64..127):
  //   records of taken nodes: rh = key high word (order-preserving score
  //     bits), rl = key low word, rs = score;
  //   frontier slots: every taken node p has at most one pending offer, its
  //     next child not yet taken, kept in slot p: kh / kl = key words,
  //     ks = its score (slots of nodes not taken yet are never read).
  // The root (node 0, score +0.0) offers its rank-0 child in slot 0.
  const float root_child = 0.0f + s_T[0];
  uint32_t rh0 = lane == 0 ? ord_f32(0.0f) : 0u, rl0 = 0u, rh1 = 0u, rl1 = 0u;
  float rs0 = 0.0f, rs1 = 0.0f;
  uint32_t kh0 = ord_f32(root_child);
  uint32_t kl0 = static_cast<uint32_t>(make_key_bits(0u, 0, 0, 1, 0));
  float ks0 = root_child;
  uint32_t kh1 = 0u, kl1 = 0u;
  float ks1 = 0.0f;
  if (lane != 0) kh0 = 0u, kl0 = 0u;

  // nodes the tree can hold: 1 + K + K^2 + ... + K^D, at most N; until that
  // many are taken the best offer is a real one
  int total = 1;
  {
    int pw = 1;
    for (int d = 1; d <= D && total < N; ++d) {
      pw = min(pw * K, N);
      total = min(total + pw, N);
    }
  }

  // What taking a slot's offer (parent p, rank r, depth d, score s) would
  // offer next: its own rank-0 child, score s + lp(d + 1, 0), and p's next
  // child, score score(p) + lp(d, r + 1).  Every lane computes both for its
  // own slot; this does not depend on the step's maximum, so it fills the
  // gaps of the maximum's dependent chain, and after the maximum a step only
  // reads the winning lane.
  auto offers = [&](uint32_t kl, float ks, float rs, float& cs, float& ss) {
    const int d = static_cast<int>((kl >> 8) & 0xFF);          // the offer's depth
    const int r1 = 256 - static_cast<int>((kl >> 16) & 0xFF);  // its rank + 1
    cs = ks + s_T[d * kRow];
    ss = rs + s_T[(d - 1) * kRow + r1];
  };

  for (int i = 1; i < total; ++i) {
    float cs0, ss0, cs1 = 0.0f, ss1 = 0.0f;
    offers(kl0, ks0, rs0, cs0, ss0);
    if (SLOTS2) offers(kl1, ks1, rs1, cs1, ss1);
    // the best slot: largest key; the high word (score) decides unless tied
    uint32_t mh = kh0, ml = kl0;
    float mcs = cs0, mss = ss0, mks = ks0;
    bool in1 = false;
    if (SLOTS2) {
      in1 = ((static_cast<uint64_t>(kh1) << 32) | kl1) > ((static_cast<uint64_t>(kh0) << 32) | kl0);
      mh = in1 ? kh1 : kh0;
      ml = in1 ? kl1 : kl0;
      mcs = in1 ? cs1 : cs0;
      mss = in1 ? ss1 : ss0;
      mks = in1 ? ks1 : ks0;
    }
    const uint32_t bh = wave_max_bcast_u32<HALF>(mh);
    const uint64_t tied = __ballot(mh == bh);
    int w = __builtin_ctzll(tied);
    if (__builtin_expect(__builtin_popcountll(tied) > 1, 0)) {
      // the cross-lane maximum runs with every lane active: written as the
      // right operand of && it would run only in the lanes where the left one
      // holds, and read stale values from the others
      const uint32_t bl = wave_max_bcast_u32<HALF>(mh == bh ? ml : 0u);
      w = __builtin_ctzll(__ballot(mh == bh && ml == bl));
    }
    // readlane yields a signed int: cast before widening, or the low word sign-extends
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(ml, w));
    const float cs = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mcs), w));
    const float ss = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mss), w));
    const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mks), w));
    const int parent = SLOTS2 ? w + 64 * (__builtin_amdgcn_readlane(in1 ? 1 : 0, w) & 1) : w;
    const int depth = static_cast<int>((lo >> 8) & 0xFF);
    // node i = the taken offer; slot i gets node i's best child, slot parent
    // the parent's next child
    const uint32_t lo_c = static_cast<uint32_t>(make_key_bits(0u, i, 0, depth + 1, i));
    const uint32_t lo_s = ((lo & 0xFFFFFF00u) - 0x10000u) | static_cast<uint32_t>(i);
    // an offer that does not exist (a child below depth D, a sibling past
    // rank K - 1) gets key 0, below every real key, -inf scores included (a
    // real log-prob may be -inf, e.g. a masked token): it is never taken
    const int rank = 255 - static_cast<int>((lo >> 16) & 0xFF);
    const uint32_t ch = depth < D ? ord_f32(cs) : 0u;
    const uint32_t sh = rank + 1 < K ? ord_f32(ss) : 0u;
    const int il = i & 63, pl = parent & 63;
    if (!TWO || i < 64) {
      rh0 = put_lane(rh0, bh, il);
      rl0 = put_lane(rl0, lo, il);
      rs0 = put_lane(rs0, sc, il);
      kh0 = put_lane(kh0, ch, il);
      kl0 = put_lane(kl0, lo_c, il);
      ks0 = put_lane(ks0, cs, il);
    } else {
      rh1 = put_lane(rh1, bh, il);
      rl1 = put_lane(rl1, lo, il);
      rs1 = put_lane(rs1, sc, il);
      kh1 = put_lane(kh1, ch, il);
      kl1 = put_lane(kl1, lo_c, il);
      ks1 = put_lane(ks1, cs, il);
    }
    if (!SLOTS2 || parent < 64) {
      kh0 = put_lane(kh0, sh, pl);
      kl0 = put_lane(kl0, lo_s, pl);
      ks0 = put_lane(ks0, ss, pl);
    } else {
      kh1 = put_lane(kh1, sh, pl);
      kl1 = put_lane(kl1, lo_s, pl);
      ks1 = put_lane(ks1, ss, pl);
    }
  }
  const int count = total;

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
    // selects rather than a computed index: a register array indexed at run
    // time would live in scratch memory
    const bool own = dep[s] >= 0, hasp = own && par[s] >= 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x = own && (i >> 5) == w ? 1u << (i & 31) : 0u;
      x |= hasp && (par[s] >> 5) == w ? 1u << (par[s] & 31) : 0u;
      va[s][w] = x;
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
  if (t.max_depth) {
    int m = max(dep[0], dep[1]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if (lane == 0) t.max_depth[b] = m;
  }
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
  const bool small_table = D * K <= 64, one_list = budget + 1 <= 64,
             one_frontier = budget + 1 <= 65, half = budget + 1 <= 33;
  const dim3 g(B), blk(kWave);
  const size_t lds = static_cast<size_t>(D + 2) * kRow * sizeof(float);
#define DDT_BUILD(R_, T_, S_, H_)                                                              \
  hipLaunchKernelGGL((build_kernel<R_, T_, S_, H_>), g, blk, lds, stream, draft_lp, draft_tok, \
                     root_tok, prefix_len, D, K, budget, *tree)
  if (small_table) {
    if (half) DDT_BUILD(1, false, false, true);
    else if (one_list) DDT_BUILD(1, false, false, false);
    else if (one_frontier) DDT_BUILD(1, true, false, false);
    else DDT_BUILD(1, true, true, false);
  } else {
    if (half) DDT_BUILD(4, false, false, true);
    else if (one_list) DDT_BUILD(4, false, false, false);
    else if (one_frontier) DDT_BUILD(4, true, false, false);
    else DDT_BUILD(4, true, true, false);
  }
#undef DDT_BUILD
  return check_launch("ddtree_build");
}
