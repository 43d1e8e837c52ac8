// Shared device helpers for the libddtree kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddtree.h"

namespace ddt {

constexpr int kWave = 64;

// ---------------------------------------------------------------- host side errors
ddtree_status fail(ddtree_status st, const char* fmt, ...);
ddtree_status check_launch(const char* what);
__host__ __device__ inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------- scalar conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Monotone map float -> uint32 (a < b  <=>  ord(a) < ord(b)); -0.0 is first
// turned into +0.0 so that the two zeros compare equal, as they do as floats.
__device__ __forceinline__ uint32_t ord_f32(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unord_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------- wave reductions
// Max over the 16 lanes of each DPP row, via quad_perm and row_ror moves.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0xB1, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x4E, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x124, 0xF, 0xF, false)));
  v = max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x128, 0xF, 0xF, false)));
  return v;
}

// Wave-uniform max of a uint32 over all 64 lanes (all lanes must be active).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row_max_u32(v);
  uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Wave-uniform max of a uint64 (lexicographic on the two halves).
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t hi = wave_max_u32(static_cast<uint32_t>(v >> 32));
  uint32_t lo = wave_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float shfl_xor_f32(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o, kWave)));
  return v;
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  return __shfl_up(v, d, kWave);
}

// Inclusive prefix sum of a uint64 across the wave (exact integer arithmetic).
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    uint64_t o = shfl_up_u64(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Wave-uniform sum of a uint64 by DPP row moves and four lane reads (all
// lanes must be active): no shuffle-index registers and no LDS round trips.
__device__ __forceinline__ uint64_t wave_sum_u64_dpp(uint64_t v) {
  uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
#define DDT_ROW_ADD(ctrl)                                                                         \
  do {                                                                                            \
    const uint32_t l2 = static_cast<uint32_t>(                                                    \
        __builtin_amdgcn_update_dpp(0, static_cast<int>(lo), ctrl, 0xF, 0xF, false));             \
    const uint32_t h2 = static_cast<uint32_t>(                                                    \
        __builtin_amdgcn_update_dpp(0, static_cast<int>(hi), ctrl, 0xF, 0xF, false));             \
    const uint64_t t = ((static_cast<uint64_t>(hi) << 32) | lo) + ((static_cast<uint64_t>(h2) << 32) | l2); \
    lo = static_cast<uint32_t>(t);                                                                \
    hi = static_cast<uint32_t>(t >> 32);                                                          \
  } while (0)
  DDT_ROW_ADD(0xB1);    // quad_perm [1, 0, 3, 2]
  DDT_ROW_ADD(0x4E);    // quad_perm [2, 3, 0, 1]
  DDT_ROW_ADD(0x124);   // row_ror 4
  DDT_ROW_ADD(0x128);   // row_ror 8
#undef DDT_ROW_ADD
  uint64_t tot = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    tot += (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(hi), 16 * r))) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(lo), 16 * r));
  return tot;
}

// ---------------------------------------------------------------- sampling weights
// Constants of the integer softmax weights for one temperature.
struct WeightConsts {
  float c;      // fp32(log2(e) / T)
  float a[7];   // fp32((ln 2)^n / n!)
};

WeightConsts weight_consts(float temperature);  // host

// w(l) = floor(p * 2^(32+k)) with y = (l - m) * c, k = rint(y), f = y - k and
// p the degree-6 Taylor polynomial of 2^f, every multiply and add rounded to
// fp32 on its own (no fused multiply-add); w = 0 when y < -32.  p * 2^24 is an
// exact integer P, so w = P * 2^(8+k), done with integer shifts.  Branch-free:
// a cut-off y is clamped to -32 for the arithmetic and its result discarded.
__device__ __forceinline__ uint64_t weight(float l, float m, const WeightConsts& wc) {
#pragma clang fp contract(off)
  const float y0 = (l - m) * wc.c;
  const bool keep = y0 >= -32.0f;
  const float y = max(y0, -32.0f);   // only the kept range matters below
  const float k = __builtin_rintf(y);
  const float f = y - k;
  float p = wc.a[6];
  p = p * f; p = p + wc.a[5];
  p = p * f; p = p + wc.a[4];
  p = p * f; p = p + wc.a[3];
  p = p * f; p = p + wc.a[2];
  p = p * f; p = p + wc.a[1];
  p = p * f; p = p + wc.a[0];
  // p in [0.7, 1.42] has at most 24 significant bits above 2^-24, so
  // P = p * 2^24 is an exact integer < 2^25, and floor(p * 2^(32 + k)) =
  // floor(P * 2^(8 + k)) = (P * 2^24) >> (16 - k) with 16 - k in [16, 48];
  // a shift of 63 gives the 0 of a dropped (y < -32) weight
  const uint32_t P = static_cast<uint32_t>(p * 16777216.0f);
  const uint32_t sh = keep ? static_cast<uint32_t>(16.0f - k) : 63u;
  const uint64_t P24 = (static_cast<uint64_t>(P >> 8) << 32) | (P << 24);
  return P24 >> sh;
}

// ---------------------------------------------------------------- weight table
// Once a row's m (and the temperature's c) are fixed, weight() of a bf16
// logit depends only on its 16-bit pattern.  A workgroup that weighs many
// logits of one row tabulates weight() in LDS for the patterns of the kTabE
// binades at and below max(|m|, |m - 32/c|) (the magnitudes that can carry
// weight), both signs: entry sign * kTabSpan + (hi - a) for the 15-bit
// magnitude pattern a in [hi - span + 1, hi], and entry 2 * kTabSpan = 0 for
// every pattern outside that window.  Callers weigh a miss with weight()
// itself, so every weight is weight()'s own value whatever the window.
constexpr int kTabE = 20;
constexpr int kTabSpan = kTabE * 128;
constexpr int kTabEntries = 2 * kTabSpan + 1;   // 40 KB of uint64

struct WeightTable {
  uint32_t hi, span;
};

// Every thread of the workgroup calls this (tid in [0, nthreads)); the caller
// synchronises the workgroup before the first lookup.
__device__ __forceinline__ WeightTable fill_weight_table(uint64_t* s_tab, float m,
                                                         const WeightConsts& wc, int tid,
                                                         int nthreads) {
  const float big = max(fabsf(m), fabsf(m - 32.0f / wc.c));
  const int e_top = static_cast<int>((__float_as_uint(big) >> 23) & 0xFFu);
  const int e_hi = min(e_top, 254), e_lo = max(e_top - kTabE + 1, 1);
  WeightTable tb;
  tb.hi = (static_cast<uint32_t>(e_hi) << 7) | 127u;
  tb.span = e_hi >= e_lo ? tb.hi - (static_cast<uint32_t>(e_lo) << 7) + 1u : 0u;
  for (int t = tid; t < kTabEntries; t += nthreads) {
    const uint32_t off = static_cast<uint32_t>(t % kTabSpan);
    uint64_t wv = 0;
    if (t < 2 * kTabSpan && off < tb.span) {
      const uint32_t u = (static_cast<uint32_t>(t / kTabSpan) << 15) | (tb.hi - off);
      const float l = __uint_as_float(u << 16);
      // patterns above m occur in no row with this maximum; their entries
      // are never read
      if (l <= m) wv = weight(l, m, wc);
    }
    s_tab[t] = wv;
  }
  return tb;
}

// Table weight of bf16 pattern u; `in` is false (and the result 0) outside
// the window.  Branch-free: a miss reads the zero entry.
__device__ __forceinline__ uint64_t table_weight(const uint64_t* s_tab, const WeightTable& tb,
                                                 uint32_t u, bool& in) {
  const uint32_t off = tb.hi - (u & 0x7FFFu);   // wraps above the window
  in = off < tb.span;
  return s_tab[in ? (u >> 15) * kTabSpan + off : 2u * kTabSpan];
}

// ---------------------------------------------------------------- greedy walk
// The greedy walk of request b by one wave ("Dissecting DDTree's
// Tree-Parallel Evaluation Strategy", Section 1 step 5): from the root, move
// to the child whose token equals the target argmax at the current node
// (children's tokens are distinct, so it is unique) until there is none or
// the depth reaches D; accept_len = moves, bonus = argmax at the last node.
// Lane l holds nodes l and l + 64 (N <= 128): their parent and token, -2 for
// nodes that do not exist.
struct WalkNodes {
  int par[2], tok[2];
};

__device__ __forceinline__ WalkNodes walk_load(const ddtree_tree& t, int b, int lane) {
  const int N = t.N;
  const long base = static_cast<long>(b) * N;
  WalkNodes w;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int j = lane + s * kWave;
    w.par[s] = j < N ? t.parent[base + j] : -2;
    w.tok[s] = j < N ? t.token[base + j] : -2;
  }
  return w;
}

// A release fence at system scope: the calling wave's earlier stores (and
// those its workgroup made before a barrier) are visible to the host before
// any of its later stores.  Release only: unlike __threadfence_system() it
// does not also invalidate the L2.
__device__ __forceinline__ void release_system() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, ""); }

// s_am: the argmax of every node of the request (-1 for padding nodes), in
// LDS; w: walk_load() with the nodes >= num_nodes[b] already set to -2.
__device__ __forceinline__ void walk_run(const ddtree_tree& t, int b, const int32_t* s_am,
                                         const WalkNodes& w, int lane,
                                         int32_t* __restrict__ accept_len,
                                         int32_t* __restrict__ path_nodes,
                                         int32_t* __restrict__ out_tokens,
                                         int32_t* __restrict__ bonus) {
  const int D = t.D;
  int32_t* path = path_nodes + static_cast<long>(b) * (D + 1);
  int32_t* outt = out_tokens + static_cast<long>(b) * (D + 1);
  int cur = 0, a = 0;
  while (a < D) {
    const int target = s_am[cur];
    const uint64_t m0 = __ballot(w.par[0] == cur && w.tok[0] == target);
    const uint64_t m1 = __ballot(w.par[1] == cur && w.tok[1] == target);
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
    bonus[b] = bon;
  }
  // accept_len last, after a system-scope release: a host that polls it in
  // mapped host memory finds the request's other outputs written
  release_system();
  if (lane == 0) accept_len[b] = a;
}

// ---------------------------------------------------------------- element access
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16 = 4;
  __device__ __forceinline__ static float get(const float* p, long i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static constexpr int kPer16 = 8;
  __device__ __forceinline__ static float get(const uint16_t* p, long i) {
    return bf16_to_f32(p[i]);
  }
};

}  // namespace ddt
