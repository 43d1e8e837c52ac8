// ddtree_tree_attention: every tree node attends to its request's context,
// read from HBM once and shared by all nodes, plus its visible tree nodes.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's
// Tree-Parallel Evaluation Strategy", Section 1 step 4 and Section 2; "The
// Pivot Point", "The Design Constraint: Load Contexts Once".
//
// Work decomposition.  For one (request b, KV head) the query tile holds all
// M = N * (Hq / Hkv) query rows (every tree node of every grouped head), so
// each context K/V tile is loaded once and serves every node.  (Past 128 rows
// the rows are cut into 128-row slices along grid z; each slice streams the
// context once.)  The context
// of request b is cut into splits of `split_keys` keys; one workgroup owns one
// (split, KV head).  The last split of a request also takes the tree keys
// (the only keys that need the visibility mask).  If a request has more than
// one split, each writes an unnormalised partial (O, running max, sum) and a
// combine kernel merges them; otherwise the split writes the output directly.
//
// Inside a workgroup (4 or 8 waves): 256 threads load one K/V tile per step
// with 16-byte coalesced loads (each thread: 4 consecutive keys of one
// 16-byte column, for K and for V) into registers, then store it to LDS --
// K row-major, V transposed -- and immediately issue the loads of the next
// tile.  Wave w < QB owns query rows [16w, 16w + 16) and computes on MFMA:
//   S^T (keys x queries) = K Q^T      (A = K from LDS, B = Q^T in registers)
//   O^T (dims x queries) += V^T P^T   (A = V^T from LDS, B = P^T, which is
//                                      exactly S^T's accumulator layout)
// with an online softmax in base 2.  bf16 uses v_mfma_f32_16x16x32_bf16,
// fp32 uses v_mfma_f32_16x16x4_f32.
#include <algorithm>
#include <cstdlib>

#include "common.hpp"

namespace ddt {

ddtree_status check_tree(const ddtree_tree* t, const char* who);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 of masked keys is 0

struct AttnArgs {
  const void* q;
  const void* k_ctx;
  const void* v_ctx;
  const int32_t* ctx_offsets;
  const void* k_tree;
  const void* v_tree;
  const uint64_t* vis;
  const int32_t* num_nodes;
  int B, N, W, Hq, Hkv, G, M;
  float scale_log2;   // scale * log2(e)
  int split_keys;
  void* out;
  float* lse;
  float* ws_o;        // [total_splits * Hkv, M, Dh] unnormalised partial outputs
  float2* ws_ml;      // [total_splits * Hkv, M] (running max in log2 units, sum)
};

// ------------------------------------------------------------------ dtype policies
// Each policy fixes: chunks of 16 bytes per K/V row (CH), LDS layout, and
// the two MFMA products.  The first 256 threads of a workgroup load the
// tiles; KT (keys per tile) = 1024 / CH so that each of them loads exactly one
// 4-key block of K and one of V per tile.

template <int DH>
struct PolicyBF16 {
  using elem = uint16_t;
  static constexpr int CH = DH * 2 / 16;
  static constexpr int QF = DH / 32;            // Q fragments (k-steps of 32)
  template <int KT> static constexpr int k_stride() { return DH + 8; }       // elements
  template <int KT> static constexpr int v_stride() { return KT + 8; }       // elements (V^T rows)
  template <int KT> static constexpr int lds_bytes() {
    return (KT * (DH + 8) + DH * (KT + 8)) * 2;
  }
  struct QFrag { bf16x8_t f[QF]; };

  __device__ __forceinline__ static void load_q(QFrag& qf, const elem* qrow, int g) {
#pragma unroll
    for (int s = 0; s < QF; ++s)
      qf.f[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 32 + 8 * g);
  }
  // store one 4-key block (keys key0..key0+3, 16-byte column e) to LDS
  template <int KT>
  __device__ __forceinline__ static void store_block(elem* k_lds, elem* vt_lds, int key0, int e, const u32x4_t (&kr)[4],
                                     const u32x4_t (&vr)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4_t*>(k_lds + (key0 + c) * k_stride<KT>() + e * 8) = kr[c];
    // V^T: within a 32-key group, key 16a + 4g + c lives at position 8g + 4a + c
    const int grp = key0 >> 5, kk = key0 & 31;
    const int pos = grp * 32 + 8 * ((kk & 15) >> 2) + 4 * (kk >> 4);
    const u32x4_t w0 = vr[0], w1 = vr[1], w2 = vr[2], w3 = vr[3];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int h = t >> 1;
      uint32_t lo, hi;
      if (t & 1) {
        lo = (w0[h] >> 16) | (w1[h] & 0xFFFF0000u);
        hi = (w2[h] >> 16) | (w3[h] & 0xFFFF0000u);
      } else {
        lo = (w0[h] & 0xFFFFu) | (w1[h] << 16);
        hi = (w2[h] & 0xFFFFu) | (w3[h] << 16);
      }
      *reinterpret_cast<u32x2_t*>(vt_lds + (e * 8 + t) * v_stride<KT>() + pos) = u32x2_t{lo, hi};
    }
  }
  // S^T block (16 keys from kbase) against this wave's 16 queries
  template <int KT>
  __device__ __forceinline__ static f32x4_t qk(const elem* k_lds, int kbase, const QFrag& qf, int l16, int g) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const elem* kp = k_lds + (kbase + l16) * k_stride<KT>() + 8 * g;
#pragma unroll
    for (int s = 0; s < QF; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8_t*>(kp + s * 32),
                                                    qf.f[s], acc, 0, 0, 0);
    return acc;
  }
  // O^T += V^T P^T over the tile; p[kb] holds the probabilities of key block kb
  template <int KT>
  __device__ __forceinline__ static void pv(const elem* vt_lds, const f32x4_t* p, f32x4_t* o, int l16, int g) {
#pragma unroll
    for (int j = 0; j < KT / 32; ++j) {
      bf16x8_t pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pf[r] = static_cast<__bf16>(p[2 * j][r]);
        pf[4 + r] = static_cast<__bf16>(p[2 * j + 1][r]);
      }
#pragma unroll
      for (int db = 0; db < DH / 16; ++db) {
        const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(
            vt_lds + (db * 16 + l16) * v_stride<KT>() + j * 32 + 8 * g);
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[db], 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ static void store_out(elem* dst, const f32x4_t& v) {
    uint32_t lo = f32_to_bf16_rne(v[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(v[1])) << 16);
    uint32_t hi = f32_to_bf16_rne(v[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(v[3])) << 16);
    *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
  }
};

template <int DH>
struct PolicyF32 {
  using elem = float;
  static constexpr int CH = DH * 4 / 16;
  static constexpr int QF = DH / 4;             // k-steps of 4
  template <int KT> static constexpr int k_stride() { return DH + 4; }
  template <int KT> static constexpr int v_stride() { return DH + 4; }
  template <int KT> static constexpr int lds_bytes() { return 2 * KT * (DH + 4) * 4; }
  struct QFrag { float f[QF]; };

  __device__ __forceinline__ static void load_q(QFrag& qf, const elem* qrow, int g) {
#pragma unroll
    for (int s = 0; s < QF; ++s) qf.f[s] = qrow[4 * s + g];
  }
  template <int KT>
  __device__ __forceinline__ static void store_block(elem* k_lds, elem* v_lds, int key0, int e, const u32x4_t (&kr)[4],
                                     const u32x4_t (&vr)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<u32x4_t*>(k_lds + (key0 + c) * k_stride<KT>() + e * 4) = kr[c];
      *reinterpret_cast<u32x4_t*>(v_lds + (key0 + c) * v_stride<KT>() + e * 4) = vr[c];
    }
  }
  template <int KT>
  __device__ __forceinline__ static f32x4_t qk(const elem* k_lds, int kbase, const QFrag& qf, int l16, int g) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const elem* kp = k_lds + (kbase + l16) * k_stride<KT>() + g;
#pragma unroll
    for (int s = 0; s < QF; ++s)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kp[4 * s], qf.f[s], acc, 0, 0, 0);
    return acc;
  }
  template <int KT>
  __device__ __forceinline__ static void pv(const elem* v_lds, const f32x4_t* p, f32x4_t* o, int l16, int g) {
#pragma unroll
    for (int kb = 0; kb < KT / 16; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const elem* vp = v_lds + (kb * 16 + 4 * g + i) * v_stride<KT>() + l16;
#pragma unroll
        for (int db = 0; db < DH / 16; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vp[db * 16], p[kb][i], o[db], 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ static void store_out(elem* dst, const f32x4_t& v) {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

// ------------------------------------------------------------------ main kernel
template <class P, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnArgs a) {
  using elem = typename P::elem;
  constexpr int DH = P::QF * (sizeof(elem) == 2 ? 32 : 4);
  constexpr int KT = 1024 / P::CH;
  constexpr int KB = KT / 16;
  static_assert(KT % 32 == 0 && KT >= 32, "tile must hold whole 32-key groups");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  elem* k_lds = reinterpret_cast<elem*>(smem);
  elem* v_lds = k_lds + KT * P::template k_stride<KT>();
  __shared__ int s_b, s_split, s_nsplit;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int sid = blockIdx.x, kvh = blockIdx.y;
  const int row0 = blockIdx.z * 128;          // query-row slice of this workgroup
  const int SK = a.split_keys;

  // which request and split this workgroup owns: prefix over per-request split counts
  if (wave == 0) {
    int acc = 0, fb = -1, fs = 0, fn = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int b = b0 + lane;
      int nb = 0;
      if (b < a.B) {
        const int L = a.ctx_offsets[b + 1] - a.ctx_offsets[b];
        nb = L > 0 ? (L + SK - 1) / SK : 1;
      }
      int incl = nb;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d, 64);
        if (lane >= d) incl += o;
      }
      const int excl = acc + incl - nb;
      if (b < a.B && sid >= excl && sid < excl + nb) {
        fb = b;
        fs = sid - excl;
        fn = nb;
      }
      acc += __shfl(incl, 63, 64);
    }
    const uint64_t hit = __ballot(fb >= 0);
    if (lane == 0) s_b = -1;
    if (hit) {
      const int src = __builtin_ctzll(hit);
      const int b = __shfl(fb, src, 64), s = __shfl(fs, src, 64), n = __shfl(fn, src, 64);
      if (lane == 0) {
        s_b = b;
        s_split = s;
        s_nsplit = n;
      }
    }
  }
  __syncthreads();
  const int b = s_b;
  if (b < 0) return;
  const int split = s_split, nsplit = s_nsplit;
  const int ctx0 = a.ctx_offsets[b];
  const int L = a.ctx_offsets[b + 1] - ctx0;
  const int k0 = split * SK, k1 = min(L, k0 + SK);
  const bool last = split == nsplit - 1;
  const int nctx_tiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  const int ntiles = nctx_tiles + (last ? (a.N + KT - 1) / KT : 0);
  const int nn = a.num_nodes[b];
  const elem* kc = static_cast<const elem*>(a.k_ctx);
  const elem* vc = static_cast<const elem*>(a.v_ctx);
  const elem* kt = static_cast<const elem*>(a.k_tree);
  const elem* vt = static_cast<const elem*>(a.v_tree);

  // this thread's 4-key block of every tile: keys 4*vq .. 4*vq+3, column e
  const bool loader = tid < 256;
  const int vq = (tid & 255) / P::CH, e = (tid & 255) % P::CH;
  u32x4_t kr[4], vr[4];
#define DDT_LOAD_KEY(c_)                                                                    \
  do {                                                                                      \
    const int key_ = min(base_ + 4 * vq + (c_), lim_ - 1);                                  \
    const long row_ = is_ctx_ ? (static_cast<long>(ctx0 + key_) * a.Hkv + kvh)              \
                              : ((static_cast<long>(b) * a.N + key_) * a.Hkv + kvh);        \
    const long off_ = row_ * DH + e * (16 / sizeof(elem));                                  \
    kr[c_] = *reinterpret_cast<const u32x4_t*>((is_ctx_ ? kc : kt) + off_);                 \
    vr[c_] = *reinterpret_cast<const u32x4_t*>((is_ctx_ ? vc : vt) + off_);                 \
  } while (0)
#define DDT_LOAD_TILE(t_)                                                                   \
  do {                                                                                      \
    const bool is_ctx_ = (t_) < nctx_tiles;                                                 \
    const int base_ = is_ctx_ ? k0 + (t_) * KT : ((t_) - nctx_tiles) * KT;                  \
    const int lim_ = is_ctx_ ? k1 : a.N;                                                    \
    DDT_LOAD_KEY(0);                                                                        \
    DDT_LOAD_KEY(1);                                                                        \
    DDT_LOAD_KEY(2);                                                                        \
    DDT_LOAD_KEY(3);                                                                        \
  } while (0)

  // query rows of this wave: r = 16*wave + l16 -> (node, head)
  const bool computes = wave < QB && row0 + 16 * wave < a.M;
  const int r = row0 + 16 * wave + l16;
  const int rq = min(r, a.M - 1);
  const int node = rq / a.G, head = kvh * a.G + rq % a.G;
  typename P::QFrag qf;
  uint64_t vis0 = 0, vis1 = 0;
  if (computes) {
    const elem* qrow = static_cast<const elem*>(a.q) +
                       ((static_cast<long>(b) * a.N + node) * a.Hq + head) * DH;
    P::load_q(qf, qrow, g);
    if (node < nn) {
      const uint64_t* vr_ = a.vis + (static_cast<long>(b) * a.N + node) * a.W;
      vis0 = vr_[0];
      vis1 = a.W > 1 ? vr_[1] : 0ull;
    }
  }
  f32x4_t o[DH / 16];
#pragma unroll
  for (int db = 0; db < DH / 16; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;

  if (ntiles > 0 && loader) DDT_LOAD_TILE(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    if (loader) {
      P::template store_block<KT>(k_lds, v_lds, 4 * vq, e, kr, vr);
      if (t + 1 < ntiles) DDT_LOAD_TILE(t + 1);
    }
    __syncthreads();
    if (!computes) continue;
    const bool is_ctx = t < nctx_tiles;
    const int base = is_ctx ? k0 + t * KT : (t - nctx_tiles) * KT;
    f32x4_t sv[KB];
    float tmax = kNegBig;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      sv[kb] = P::template qk<KT>(k_lds, kb * 16, qf, l16, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = base + kb * 16 + 4 * g + i;
        bool ok;
        if (is_ctx) {
          ok = key < k1;
        } else {
          const uint64_t w = key < 64 ? vis0 : vis1;
          ok = key < a.N && ((w >> (key & 63)) & 1ull);
        }
        const float sc = ok ? sv[kb][i] * a.scale_log2 : -__builtin_huge_valf();
        sv[kb][i] = sc;
        tmax = max(tmax, sc);
      }
    }
    tmax = max(tmax, shfl_xor_f32(tmax, 16));
    tmax = max(tmax, shfl_xor_f32(tmax, 32));
    const float m_new = max(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(sv[kb][i] - m_new);
        sv[kb][i] = pv;
        psum += pv;
      }
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) o[db] *= alpha;
    P::template pv<KT>(v_lds, sv, o, l16, g);
  }
#undef DDT_LOAD_TILE
#undef DDT_LOAD_KEY
  if (!computes) return;

  float l_tot = l_run + shfl_xor_f32(l_run, 16);
  l_tot += shfl_xor_f32(l_tot, 32);
  if (r >= a.M) return;
  if (nsplit == 1) {
    elem* orow = static_cast<elem*>(a.out) + ((static_cast<long>(b) * a.N + node) * a.Hq + head) * DH;
    const bool valid = node < nn;
    const float inv = valid && l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db) P::store_out(orow + db * 16 + 4 * g, o[db] * inv);
    if (a.lse && g == 0)
      a.lse[(static_cast<long>(b) * a.N + node) * a.Hq + head] =
          valid ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_huge_valf();
  } else {
    const long pr = (static_cast<long>(sid) * a.Hkv + kvh) * a.M + r;
    float* dst = a.ws_o + pr * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
      *reinterpret_cast<float4*>(dst + db * 16 + 4 * g) =
          make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g == 0) a.ws_ml[pr] = make_float2(m_run, l_tot);
  }
}

// ------------------------------------------------------------------ combine
template <typename elem, int DH>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  const int b = blockIdx.x, kvh = blockIdx.y;
  const int SK = a.split_keys;
  auto nsplits = [&](int bb) {
    const int L = a.ctx_offsets[bb + 1] - a.ctx_offsets[bb];
    return L > 0 ? (L + SK - 1) / SK : 1;
  };
  const int ns = nsplits(b);
  if (ns == 1) return;
  int start = 0;
  for (int bb = 0; bb < b; ++bb) start += nsplits(bb);
  const int nn = a.num_nodes[b];
  constexpr int TPR = DH / 4;                 // threads per row, 4 dims each
  constexpr int RPI = 256 / TPR;              // rows per iteration
  const int sub = threadIdx.x / TPR, d4 = (threadIdx.x % TPR) * 4;
  for (int r = sub; r < a.M; r += RPI) {
    const int node = r / a.G, head = kvh * a.G + r % a.G;
    const long orow = ((static_cast<long>(b) * a.N + node) * a.Hq + head);
    elem* dst = static_cast<elem*>(a.out) + orow * DH + d4;
    if (node >= nn) {
      if constexpr (sizeof(elem) == 2) *reinterpret_cast<uint2*>(dst) = make_uint2(0u, 0u);
      else *reinterpret_cast<float4*>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
      if (a.lse && d4 == 0) a.lse[orow] = -__builtin_huge_valf();
      continue;
    }
    float mstar = kNegBig;
    for (int s = 0; s < ns; ++s)
      mstar = max(mstar, a.ws_ml[(static_cast<long>(start + s) * a.Hkv + kvh) * a.M + r].x);
    float lsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
      const long pr = (static_cast<long>(start + s) * a.Hkv + kvh) * a.M + r;
      const float2 ml = a.ws_ml[pr];
      const float w = __builtin_amdgcn_exp2f(ml.x - mstar);
      lsum += w * ml.y;
      const float4 v = *reinterpret_cast<const float4*>(a.ws_o + pr * DH + d4);
      acc.x += w * v.x;
      acc.y += w * v.y;
      acc.z += w * v.z;
      acc.w += w * v.w;
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    if constexpr (sizeof(elem) == 2) {
      const uint32_t lo = f32_to_bf16_rne(acc.x * inv) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.y * inv)) << 16);
      const uint32_t hi = f32_to_bf16_rne(acc.z * inv) | (static_cast<uint32_t>(f32_to_bf16_rne(acc.w * inv)) << 16);
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(dst) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    if (a.lse && d4 == 0) a.lse[orow] = (mstar + __log2f(lsum)) * kLn2;
  }
}

// ------------------------------------------------------------------ host side
int keys_per_tile(ddtree_dtype dt, int Dh, int /*qb*/) {
  const int ch = Dh * (dt == DDTREE_BF16 ? 2 : 4) / 16;
  return 1024 / ch;
}

// Keys per split: about `target` workgroups over the whole context, whole tiles.
int plan_split_keys(const int32_t* offs_host, int B, int Hkv, int kt) {
  long total = static_cast<long>(offs_host[B]) - offs_host[0];
  int target = 768;
  if (const char* env = std::getenv("DDTREE_ATTN_TARGET_WGS")) target = std::max(1, atoi(env));
  long sk = (total * Hkv + target - 1) / target;
  sk = std::max<long>(sk, 2 * kt);
  sk = (sk + kt - 1) / kt * kt;
  if (const char* env = std::getenv("DDTREE_ATTN_SPLIT_KEYS")) {
    const long v = atol(env);
    if (v > 0) sk = (v + kt - 1) / kt * kt;
  }
  return static_cast<int>(std::min<long>(sk, 1L << 30));
}

int count_splits(const int32_t* offs_host, int B, int sk, bool* any_multi) {
  int tot = 0;
  *any_multi = false;
  for (int b = 0; b < B; ++b) {
    const int L = offs_host[b + 1] - offs_host[b];
    const int nb = L > 0 ? (L + sk - 1) / sk : 1;
    *any_multi |= nb > 1;
    tot += nb;
  }
  return tot;
}

template <class P, int QB>
void launch_main(const AttnArgs& a, int total_splits, hipStream_t st) {
  constexpr int NW = QB <= 4 ? 4 : 8;
  constexpr int KT = 1024 / P::CH;
  const size_t lds = P::template lds_bytes<KT>();
  const dim3 grid(total_splits, a.Hkv, (a.M + 127) / 128);
  hipLaunchKernelGGL((attn_kernel<P, QB, NW>), grid, dim3(NW * 64), lds, st, a);
}

template <class P>
void launch_qb(int qb, const AttnArgs& a, int total_splits, hipStream_t st) {
  switch (qb) {
    case 1: launch_main<P, 1>(a, total_splits, st); break;
    case 2: launch_main<P, 2>(a, total_splits, st); break;
    case 3: launch_main<P, 3>(a, total_splits, st); break;
    case 4: launch_main<P, 4>(a, total_splits, st); break;
    case 5: launch_main<P, 5>(a, total_splits, st); break;
    case 6: launch_main<P, 6>(a, total_splits, st); break;
    case 7: launch_main<P, 7>(a, total_splits, st); break;
    default: launch_main<P, 8>(a, total_splits, st); break;
  }
}

}  // namespace
}  // namespace ddt

extern "C" size_t ddtree_tree_attention_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                                       int32_t Hkv, int32_t Dh,
                                                       const int32_t* ctx_offsets_host) {
  using namespace ddt;
  if (B < 1 || N < 1 || Hkv < 1 || Hq % Hkv != 0 || !ctx_offsets_host || (Dh != 64 && Dh != 128))
    return 0;
  const int M = N * (Hq / Hkv);
  const int qb = (M + 15) / 16;
  size_t best = 0;
  for (ddtree_dtype dt : {DDTREE_BF16, DDTREE_F32}) {
    const int sk = plan_split_keys(ctx_offsets_host, B, Hkv, keys_per_tile(dt, Dh, qb));
    bool multi;
    const int tot = count_splits(ctx_offsets_host, B, sk, &multi);
    if (!multi) continue;
    const size_t need = static_cast<size_t>(tot) * Hkv * M * (Dh * sizeof(float) + sizeof(float2));
    best = std::max(best, need);
  }
  return best;
}

extern "C" ddtree_status ddtree_tree_attention(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_offsets,
    const int32_t* ctx_offsets_host, const void* k_tree, const void* v_tree,
    const ddtree_tree* tree, int32_t Hq, int32_t Hkv, int32_t Dh, ddtree_dtype dtype,
    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_tree_attention");
  if (st != DDTREE_OK) return st;
  if (!q || !k_tree || !v_tree || !ctx_offsets || !ctx_offsets_host || !out)
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: null pointer");
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: unknown dtype %d", static_cast<int>(dtype));
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: Hq=%d must be a multiple of Hkv=%d", Hq, Hkv);
  if (Dh != 64 && Dh != 128)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_tree_attention: head_dim %d (supported: 64, 128)", Dh);
  if (!(scale > 0.0f) || !(scale < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: scale must be > 0 and finite");
  const int B = tree->B, N = tree->N;
  const int M = N * (Hq / Hkv);
  if (M > 1024)
    return fail(DDTREE_EUNSUPPORTED,
                "ddtree_tree_attention: %d query rows per KV head (N * Hq / Hkv) exceed 1024", M);
  if (ctx_offsets_host[0] != 0)
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: ctx_offsets[0] must be 0");
  for (int b = 0; b < B; ++b)
    if (ctx_offsets_host[b + 1] < ctx_offsets_host[b])
      return fail(DDTREE_EINVAL, "ddtree_tree_attention: ctx_offsets must be non-decreasing");
  if (ctx_offsets_host[B] > 0 && (!k_ctx || !v_ctx))
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: null context K/V");
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
      (k_ctx && !aligned16(k_ctx)) || (v_ctx && !aligned16(v_ctx)))
    return fail(DDTREE_EINVAL, "ddtree_tree_attention: tensors must be 16-byte aligned");
  const int qb = (std::min(M, 128) + 15) / 16;   // 16-row query blocks per slice
  const int kt = keys_per_tile(dtype, Dh, qb);
  const int sk = plan_split_keys(ctx_offsets_host, B, Hkv, kt);
  bool multi;
  const int total = count_splits(ctx_offsets_host, B, sk, &multi);
  AttnArgs a;
  a.q = q;
  a.k_ctx = k_ctx;
  a.v_ctx = v_ctx;
  a.ctx_offsets = ctx_offsets;
  a.k_tree = k_tree;
  a.v_tree = v_tree;
  a.vis = tree->vis;
  a.num_nodes = tree->num_nodes;
  a.B = B;
  a.N = N;
  a.W = tree->W;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.M = M;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.split_keys = sk;
  a.out = out;
  a.lse = lse;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  if (multi) {
    const size_t need = static_cast<size_t>(total) * Hkv * M * Dh * sizeof(float);
    const size_t need_ml = static_cast<size_t>(total) * Hkv * M * sizeof(float2);
    if (!workspace || workspace_bytes < need + need_ml || !aligned16(workspace))
      return fail(DDTREE_EINVAL, "ddtree_tree_attention: workspace of %zu bytes needed, got %zu",
                  need + need_ml, workspace_bytes);
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + need);
  }
  if (dtype == DDTREE_BF16) {
    if (Dh == 128) launch_qb<PolicyBF16<128>>(qb, a, total, stream);
    else launch_qb<PolicyBF16<64>>(qb, a, total, stream);
  } else {
    if (Dh == 128) launch_qb<PolicyF32<128>>(qb, a, total, stream);
    else launch_qb<PolicyF32<64>>(qb, a, total, stream);
  }
  if (multi) {
    const dim3 g(B, Hkv);
    if (dtype == DDTREE_BF16) {
      if (Dh == 128) hipLaunchKernelGGL((combine_kernel<uint16_t, 128>), g, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((combine_kernel<uint16_t, 64>), g, dim3(256), 0, stream, a);
    } else {
      if (Dh == 128) hipLaunchKernelGGL((combine_kernel<float, 128>), g, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL((combine_kernel<float, 64>), g, dim3(256), 0, stream, a);
    }
  }
  return check_launch("ddtree_tree_attention");
}
