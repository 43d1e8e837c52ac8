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
// Inside a workgroup (4 or 8 waves).  bf16 at head_dim 128 (attn_dma_kernel):
// the K and V tiles go from global memory straight into a ring of LDS stages
// (global_load_lds, rows XOR-swizzled), the next tiles' loads in flight while
// the current one is used; V^T fragments come from transposing LDS reads.
// fp32 and head_dim 64 (attn_kernel): 256 threads load one K/V tile per step
// with 16-byte coalesced loads (each thread: 4 consecutive keys of one
// 16-byte column, for K and for V) into registers, then store it to LDS --
// K row-major, V transposed -- and immediately issue the loads of the next
// tile.  Either way wave w < QB owns query rows [16w, 16w + 16) and computes
// on MFMA:
//   S^T (keys x queries) = K Q^T      (A = K from LDS, B = Q^T in registers)
//   O^T (dims x queries) += V^T P^T   (A = V^T from LDS, B = P^T, which is
//                                      exactly S^T's accumulator layout)
// with an online softmax in base 2.  bf16 uses v_mfma_f32_16x16x32_bf16,
// fp32 uses v_mfma_f32_16x16x4_f32.
//
// The split plan comes from host copies of the context lengths; the capped
// range form plans from host upper bounds and reads the lengths themselves
// from device memory when the kernels run (splits past a request's length
// exit at once), so that one captured call serves growing caches.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "common.hpp"

// Split partials of ddtree_tree_attention_noalloc: a device array of fixed
// size in place of a caller workspace (each GPU holds its own copy until the
// process ends).  Its name in host code is only a stand-in: host code uses the
// device address that scratch_address() looks up.
static __device__ __align__(256) unsigned char scratch[DDTREE_NOALLOC_SCRATCH_BYTES];

namespace ddt {

ddtree_status check_tree(const ddtree_tree* t, const char* who);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 of masked keys is 0

// Requests whose split plan travels in the kernel arguments (about 0.8 KB of
// table); larger batches look their splits up on the device.
constexpr int kTabMax = 64;

struct AttnArgs {
  const void* q;
  const void* k_ctx;
  const void* v_ctx;
  const int32_t* ctx_offsets;   // [B+1] packed context ranges, or null when ctx_start is set
  const int32_t* ctx_start;     // [B] first context row of each request (range form), or null
  const int32_t* ctx_len;       // [B] context length of each request (range form)
  const void* k_tree;
  const void* v_tree;
  const uint64_t* vis;
  const int32_t* num_nodes;
  int B, N, W, Hq, Hkv, G, M;
  float scale_log2;   // scale * log2(e)
  int split_keys;
  int total_splits;   // splits of the host plan: the grid's x extent and the rows of ws_o / ws_ml
  void* out;
  float* lse;
  void* ws_o;         // [total_splits * Hkv, M, Dh] unnormalised partial outputs
                      // (bf16 from the DMA kernel, fp32 from the register kernel)
  float2* ws_ml;      // [total_splits * Hkv, M] (running max in log2 units, sum)
  // split plan for B <= kTabMax (tab_n = B, else 0): request b owns splits
  // [tab_split0[b], tab_split0[b+1]) and context rows [tab_off[b], tab_off[b] + tab_len[b]).
  // With the table the kernels never read the device context arrays, so the
  // host copies alone decide what is read.
  int tab_n;
  int tab_split0[kTabMax + 1];
  int tab_off[kTabMax];
  int tab_len[kTabMax];
  // capped form (ddtree_tree_attention_ranges_capped): tab_len holds upper
  // bounds that fix the plan; the kernels read the lengths from ctx_len when
  // they run, take the splits those lengths need and leave the rest idle
  int dyn_len;
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
  __device__ __forceinline__ static void store_block(elem* k_lds, elem* vt_lds, int key0, int e,
                                                     int vkey0, int ve, const u32x4_t (&kr)[4],
                                                     const u32x4_t (&vr)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4_t*>(k_lds + (key0 + c) * k_stride<KT>() + e * 8) = kr[c];
    // V^T: within a 32-key group, key 16a + 4g + c lives at position 8g + 4a + c
    const int grp = vkey0 >> 5, kk = vkey0 & 31;
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
      *reinterpret_cast<u32x2_t*>(vt_lds + (ve * 8 + t) * v_stride<KT>() + pos) = u32x2_t{lo, hi};
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
  __device__ __forceinline__ static void store_block(elem* k_lds, elem* v_lds, int key0, int e,
                                                     int vkey0, int ve, const u32x4_t (&kr)[4],
                                                     const u32x4_t (&vr)[4]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      *reinterpret_cast<u32x4_t*>(k_lds + (key0 + c) * k_stride<KT>() + e * 4) = kr[c];
      *reinterpret_cast<u32x4_t*>(v_lds + (vkey0 + c) * v_stride<KT>() + ve * 4) = vr[c];
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

// ------------------------------------------------------------------ split lookup
// Work item of a workgroup: request b, split index and count, context range.
struct SplitItem {
  int b, split, nsplit, ctx0, len;
};

// Context rows of request bb: [*off, *off + *L), from the packed offsets or
// from the per-request (start, length) ranges.
__device__ __forceinline__ void ctx_range(const AttnArgs& a, int bb, int* off, int* L) {
  if (a.ctx_start) {
    *off = a.ctx_start[bb];
    *L = a.ctx_len[bb];
  } else {
    *off = a.ctx_offsets[bb];
    *L = a.ctx_offsets[bb + 1] - *off;
  }
}

// Which request owns split `sid` (splits are numbered request by request,
// ceil(L_b / SK) of them, at least one).  For up to kTabMax requests the host
// passes the split plan and context ranges in the kernel arguments; otherwise
// wave 0 searches the context ranges and publishes the result in LDS.
__device__ __forceinline__ void find_split(const AttnArgs& a, int sid, int SK, int lane,
                                           SplitItem* out);

__device__ __forceinline__ SplitItem lookup_split(const AttnArgs& a, int sid, int wave, int lane,
                                                  SplitItem* shared_item) {
  if (a.tab_n > 0) {
    if (sid >= a.tab_split0[a.tab_n]) return SplitItem{-1, 0, 0, 0, 0};
    // the last request whose first split is <= sid (every request has one)
    int lo = 0, hi = a.tab_n;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.tab_split0[mid] <= sid) lo = mid; else hi = mid;
    }
    SplitItem it{lo, sid - a.tab_split0[lo], a.tab_split0[lo + 1] - a.tab_split0[lo],
                 a.tab_off[lo], a.tab_len[lo]};
    if (a.dyn_len) {
      // the length now in device memory, clamped to the planned bound
      it.len = min(max(a.ctx_len[lo], 0), a.tab_len[lo]);
      it.nsplit = it.len > 0 ? (it.len + a.split_keys - 1) / a.split_keys : 1;
      if (it.split >= it.nsplit) it.b = -1;   // a split past the context: idle
    }
    return it;
  }
  if (wave == 0) find_split(a, sid, a.split_keys, lane, shared_item);
  __syncthreads();
  return *shared_item;
}

__device__ __forceinline__ void find_split(const AttnArgs& a, int sid, int SK, int lane,
                                           SplitItem* out) {
  int acc = 0, fb = -1, fs = 0, fn = 0, fo = 0, fl = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int bb = b0 + lane;
    int nb = 0, off = 0, L = 0;
    if (bb < a.B) {
      ctx_range(a, bb, &off, &L);
      nb = L > 0 ? (L + SK - 1) / SK : 1;
    }
    int incl = nb;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    const int excl = acc + incl - nb;
    if (bb < a.B && sid >= excl && sid < excl + nb) {
      fb = bb;
      fs = sid - excl;
      fn = nb;
      fo = off;
      fl = L;
    }
    acc += __shfl(incl, 63, 64);
  }
  const uint64_t hit = __ballot(fb >= 0);
  if (lane == 0) out->b = -1;
  if (hit) {
    const int src = __builtin_ctzll(hit);
    const int bb = __shfl(fb, src, 64), ss = __shfl(fs, src, 64), nn = __shfl(fn, src, 64);
    const int oo = __shfl(fo, src, 64), ll = __shfl(fl, src, 64);
    if (lane == 0) *out = SplitItem{bb, ss, nn, oo, ll};
  }
}

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
  __shared__ SplitItem s_item;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int sid = blockIdx.x, kvh = blockIdx.y;
  const int row0 = blockIdx.z * 128;          // query-row slice of this workgroup
  const int SK = a.split_keys;

  const SplitItem it = lookup_split(a, sid, wave, lane, &s_item);
  const int b = it.b;
  if (b < 0) return;
  const int split = it.split, nsplit = it.nsplit;
  const int ctx0 = it.ctx0;
  const int L = it.len;
  const int k0 = split * SK, k1 = min(L, k0 + SK);
  const bool last = split == nsplit - 1;
  const int nctx_tiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  const int ntiles = nctx_tiles + (last ? (a.N + KT - 1) / KT : 0);
  const int nn = a.num_nodes[b];
  const elem* kc = static_cast<const elem*>(a.k_ctx);
  const elem* vc = static_cast<const elem*>(a.v_ctx);
  const elem* kt = static_cast<const elem*>(a.k_tree);
  const elem* vt = static_cast<const elem*>(a.v_tree);

  // this thread's 4-key blocks of every tile: keys 4*q .. 4*q+3 of 16-byte column e.
  // K: column fastest (a row is read whole, LDS rows written whole).  V: key quad
  // fastest, so that the transposed LDS writes of one instruction land in one row.
  const bool loader = tid < 256;
  const int vq = (tid & 255) / P::CH, e = (tid & 255) % P::CH;
  const int vq_v = (tid & 255) % (KT / 4), e_v = (tid & 255) / (KT / 4);
  u32x4_t kr[4], vr[4];
#define DDT_ROW(q_, c_)                                                                     \
  (is_ctx_ ? (static_cast<long>(ctx0 + min(base_ + 4 * (q_) + (c_), lim_ - 1)) * a.Hkv + kvh) \
           : ((static_cast<long>(b) * a.N + min(base_ + 4 * (q_) + (c_), lim_ - 1)) * a.Hkv + kvh))
#define DDT_LOAD_KEY(c_)                                                                    \
  do {                                                                                      \
    kr[c_] = *reinterpret_cast<const u32x4_t*>((is_ctx_ ? kc : kt) + DDT_ROW(vq, c_) * DH + \
                                               e * (16 / sizeof(elem)));                    \
    vr[c_] = *reinterpret_cast<const u32x4_t*>((is_ctx_ ? vc : vt) +                        \
                                               DDT_ROW(vq_v, c_) * DH +                     \
                                               e_v * (16 / sizeof(elem)));                  \
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
      P::template store_block<KT>(k_lds, v_lds, 4 * vq, e, 4 * vq_v, e_v, kr, vr);
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
#undef DDT_ROW
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
    float* dst = static_cast<float*>(a.ws_o) + pr * DH;
#pragma unroll
    for (int db = 0; db < DH / 16; ++db)
      *reinterpret_cast<float4*>(dst + db * 16 + 4 * g) =
          make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g == 0) a.ws_ml[pr] = make_float2(m_run, l_tot);
  }
}

// ------------------------------------------------------------------ DMA pipeline (bf16, Dh 128)
// The same computation as attn_kernel, with the context streamed by the
// global->LDS DMA path of gfx950 (global_load_lds_dwordx4: each lane's 16 bytes
// land at M0 + 16 * lane) into a ring of NS tile buffers, so that NS - 1 tiles
// are in flight while one is computed and no registers are spent on staging.
// Rows are stored whole (256 bytes) with their sixteen 16-byte chunks XOR-
// swizzled by the row index (kSwK / kSwV below), which spreads the DMA writes
// and the MFMA operand reads over the LDS banks.  V stays row-major: the V^T operand of the
// PV product comes from ds_read_b64_tr_b16, whose 16-lane transpose yields, for
// lane (g, i), V[4g + k][d0 + i] (k = 0..3) when lane j of the 16 points at
// row 4g + j/4, column d0 + 4 (j % 4) -- exactly the key order of the S^T
// accumulator.  The DMA is issued from inline asm with explicit vmcnt waits,
// because the compiler's own tracking would wait for every DMA before each
// LDS read.  Per tile, only the last context tile of a split and the tree
// tiles are masked, and the running maximum may lag (kLagLog2), so the common
// tile is two MFMA products, one cross-row max, the exponentials and one
// accumulation.

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ void dma16(const void* g, uint32_t lds_byte) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_byte);   // wave-uniform by construction
  // M0 written by a scalar move needs one wait state before an LDS-DMA load
  // reads it.  M0 is a reserved register the compiler does not allocate; no
  // other code of these kernels relies on its contents.
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m0v), "v"(g)
               : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// NaN-propagating maximum: gfx950 has a three-operand instruction for it that,
// unlike fmaxf's, needs no quieting of its operands first
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48): the gfx950
// lane swaps return {x, x of the partner lane} in some order
__device__ __forceinline__ float rows_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return nmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Rows keep a running maximum that may lag the true one by up to this many
// log2 units: the accumulators are rescaled only when a score exceeds it by
// more, so p = 2^(s - m) stays <= 2^8 and the rescale is rare.
constexpr float kLagLog2 = 8.0f;

// XOR swizzle masks of the LDS rows: a 64-lane ds_read_b128 is served 16 lanes
// (256 bytes, all 64 banks) at a time, and the K reads' 16 lanes are 16
// consecutive rows, so K rows swizzle by (row & 15) (with (row & 7), rows r and
// r + 8 collided: measured 2.7 conflict cycles per LDS instruction, 1.3 now).
// The V reads' lane groups span 8 rows; (row & 15) measured no different there.
constexpr int kSwK = 15, kSwV = 7;

template <int QB, int NW, int NS>
__global__ __launch_bounds__(NW * 64) void attn_dma_kernel(AttnArgs a) {
  using elem = uint16_t;
  constexpr int DH = 128, KT = 64, KB = KT / 16, QF = DH / 32, DB = DH / 16;
  constexpr int HALF = KT * DH * 2;               // 16 KB: the K (or V) rows of a tile
  constexpr int TILE = 2 * HALF;
  constexpr int DPW = 32 / NW;                    // 1 KB DMA instructions per wave per tile
  constexpr bool kHoist = NW == 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  __shared__ SplitItem s_item;
  const uint32_t smem_base = static_cast<uint32_t>(reinterpret_cast<size_t>(
      (__attribute__((address_space(3))) unsigned char*)(smem)));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int sid = blockIdx.x, kvh = blockIdx.y;
  const int row0 = blockIdx.z * 128;
  const int SK = a.split_keys;

  const SplitItem it = lookup_split(a, sid, wave, lane, &s_item);
  const int b = it.b;
  if (b < 0) return;
  const int k0 = it.split * SK, k1 = min(it.len, k0 + SK);
  const bool last = it.split == it.nsplit - 1;
  const int nctx_tiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  const int ntiles = nctx_tiles + (last ? (a.N + KT - 1) / KT : 0);

  // DMA of tile t into ring slot t % NS: this wave's DPW groups of four rows
  // (groups 0..15 are K rows, 16..31 V rows)
  const int rstride = a.Hkv * DH;   // elements between consecutive keys
  const elem* kc0 = static_cast<const elem*>(a.k_ctx) + (static_cast<long>(it.ctx0) * a.Hkv + kvh) * DH;
  const elem* vc0 = static_cast<const elem*>(a.v_ctx) + (static_cast<long>(it.ctx0) * a.Hkv + kvh) * DH;
  const elem* kt0 = static_cast<const elem*>(a.k_tree) + (static_cast<long>(b) * a.N * a.Hkv + kvh) * DH;
  const elem* vt0 = static_cast<const elem*>(a.v_tree) + (static_cast<long>(b) * a.N * a.Hkv + kvh) * DH;
  const int lrow = lane >> 4, lchunk = lane & 15;
  int loff[DPW];
#pragma unroll
  for (int j = 0; j < DPW; ++j) {
    const int r = 4 * ((wave * DPW + j) & 15) + lrow;
    loff[j] = r * rstride + ((lchunk ^ (r & ((wave * DPW + j) >> 4 ? kSwV : kSwK))) * 8);
  }
#define DDT_DMA_TILE(T_)                                                                        \
  do {                                                                                          \
    const int t_ = (T_);                                                                        \
    const bool ctx_ = t_ < nctx_tiles;                                                          \
    const int base_ = ctx_ ? k0 + t_ * KT : (t_ - nctx_tiles) * KT;                             \
    const int lim_ = (ctx_ ? k1 : a.N) - 1;                                                     \
    const uint32_t slot_ = smem_base + static_cast<uint32_t>((t_ % NS) * TILE);                 \
    if (base_ + KT - 1 <= lim_) {                                                               \
      _Pragma("unroll") for (int j_ = 0; j_ < DPW; ++j_) {                                      \
        const int rg_ = wave * DPW + j_;                                                        \
        const elem* p_ = (rg_ >> 4 ? (ctx_ ? vc0 : vt0) : (ctx_ ? kc0 : kt0)) +                 \
                         static_cast<long>(base_) * rstride;                                    \
        dma16(p_ + loff[j_], slot_ + static_cast<uint32_t>((rg_ >> 4) * HALF + (rg_ & 15) * 1024)); \
      }                                                                                         \
    } else {                                                                                    \
      _Pragma("unroll") for (int j_ = 0; j_ < DPW; ++j_) {                                      \
        const int rg_ = wave * DPW + j_;                                                        \
        const int vp_ = rg_ >> 4, rq_ = rg_ & 15;                                               \
        const int r_ = 4 * rq_ + lrow;                                                          \
        const int key_ = min(base_ + r_, lim_);                                                 \
        const elem* src_ = (vp_ ? (ctx_ ? vc0 : vt0) : (ctx_ ? kc0 : kt0)) +                    \
                           static_cast<long>(key_) * rstride +                                  \
                           ((lchunk ^ (r_ & (vp_ ? kSwV : kSwK))) * 8);                         \
        dma16(src_, slot_ + static_cast<uint32_t>(vp_ * HALF + rq_ * 1024));                    \
      }                                                                                         \
    }                                                                                           \
  } while (0)

  // The first NS - 1 tiles go out before anything else is read, so that their
  // latency overlaps that of the query and visibility loads below.
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < ntiles) DDT_DMA_TILE(t);

  const int nn = a.num_nodes[b];
  const bool computes = wave < QB && row0 + 16 * wave < a.M;
  const int r = row0 + 16 * wave + l16;
  const int rq = min(r, a.M - 1);
  const int node = rq / a.G, head = kvh * a.G + rq % a.G;
  bf16x8_t qf[QF];
  uint64_t vis0 = 0, vis1 = 0;
  if (computes) {
    const elem* qrow = static_cast<const elem*>(a.q) +
                       ((static_cast<long>(b) * a.N + node) * a.Hq + head) * DH;
#pragma unroll
    for (int s = 0; s < QF; ++s) qf[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 32 + 8 * g);
    if (node < nn) {
      const uint64_t* vr_ = a.vis + (static_cast<long>(b) * a.N + node) * a.W;
      vis0 = vr_[0];
      vis1 = a.W > 1 ? vr_[1] : 0ull;
    }
  }
  // Wait for all of it (the prologue tiles included): afterwards the only
  // loads in flight are the DMAs counted below.  The builtin form lets the
  // compiler's own wait tracking see this wait.
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

  f32x4_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;
  const float c = a.scale_log2;

  for (int t = 0; t < ntiles; ++t) {
    // tiles issued after t and possibly still in flight: min(ntiles - 1, t + NS - 2) - t
    const int after = min(ntiles - 1, t + NS - 2) - t;
    if (after >= 2) wait_vmcnt<2 * DPW>();
    else if (after == 1) wait_vmcnt<DPW>();
    else wait_vmcnt<0>();
    // a barrier that LDS reads of this tile cannot be moved above
    asm volatile("s_barrier" ::: "memory");
    if (t + NS - 1 < ntiles) DDT_DMA_TILE(t + NS - 1);
    if (!computes) continue;
    const unsigned char* kbuf = smem + (t % NS) * TILE;
    const unsigned char* vbuf = kbuf + HALF;
    f32x4_t sv[KB];
    bf16x8_t vf[kHoist ? KT / 32 : 1][kHoist ? DB : 1];
    if constexpr (kHoist) {
      // With 4 waves (at most two per SIMD), every LDS read of the tile is
      // issued ahead of its use, so that a wave keeps many reads in flight
      // instead of waiting on each: all K fragments, then the QK^T products,
      // then all V^T fragments, whose latency the softmax below covers.  The
      // scheduling barriers keep the compiler from interleaving each read with
      // its consumer again.  (This needs ~210 VGPRs; the 8-wave form must stay
      // at <= 128 so that two of its workgroups share a CU, and keeps the
      // compiler's own schedule.)  K fragments and products go k-step by
      // k-step, so the KB independent accumulator chains interleave.
      bf16x8_t kf[QF][KB];
#pragma unroll
      for (int s = 0; s < QF; ++s)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int row = kb * 16 + l16;
          kf[s][kb] = *reinterpret_cast<const bf16x8_t*>(
              kbuf + row * (DH * 2) + (((4 * s + g) ^ (row & kSwK)) * 16));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) sv[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < QF; ++s)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          sv[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[s][kb], qf[s], sv[kb], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < KT / 32; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          i16x4_t h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = 32 * j + 16 * hh + 4 * g + (l16 >> 2);
            const int chunk = 2 * db + ((l16 & 3) >> 1);
            const unsigned char* p = vbuf + row * (DH * 2) + ((chunk ^ (row & kSwV)) * 16) + (l16 & 1) * 8;
            h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
          }
          // whole-vector casts: element-wise bf16 inserts from the 16-bit lanes
          // are lowered wrongly (the upper half of each read is dropped)
          const u32x2_t w0 = __builtin_bit_cast(u32x2_t, h[0]);
          const u32x2_t w1 = __builtin_bit_cast(u32x2_t, h[1]);
          vf[j][db] = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
        }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const int row = kb * 16 + l16;
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < QF; ++s) {
          const bf16x8_t kf = *reinterpret_cast<const bf16x8_t*>(
              kbuf + row * (DH * 2) + (((4 * s + g) ^ (row & kSwK)) * 16));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], acc, 0, 0, 0);
        }
        sv[kb] = acc;
      }
    }
    // masks: only the last context tile of a split and the tree tiles have any
    if (!(t < nctx_tiles && k0 + (t + 1) * KT <= k1)) {
      uint64_t mask;
      if (t < nctx_tiles) {
        const int n = k1 - (k0 + t * KT);   // < 64 here
        mask = (1ull << n) - 1ull;
      } else {
        mask = t == nctx_tiles ? vis0 : vis1;
      }
      const uint64_t mg = mask >> (4 * g);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!((mg >> (kb * 16 + e)) & 1ull)) sv[kb][e] = -__builtin_huge_valf();
    }
    // online softmax in base 2 with a lagging maximum
    float t0 = nmax(nmax(sv[0][0], sv[0][1]), nmax(sv[0][2], sv[0][3]));
#pragma unroll
    for (int kb = 1; kb < KB; ++kb)
      t0 = nmax(t0, nmax(nmax(sv[kb][0], sv[kb][1]), nmax(sv[kb][2], sv[kb][3])));
    const float mc = rows_max(t0) * c;
    const bool up = mc > m_run + kLagLog2;
    if (__builtin_amdgcn_ballot_w64(up)) {
      const float m_new = up ? mc : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[kb][e], c, -m_run));
        sv[kb][e] = pv;
        psum += pv;
      }
    l_run += psum;
#pragma unroll
    for (int j = 0; j < KT / 32; ++j) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = static_cast<__bf16>(sv[2 * j][e]);
        pf[4 + e] = static_cast<__bf16>(sv[2 * j + 1][e]);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x8_t v8;
        if constexpr (kHoist) {
          v8 = vf[j][db];
        } else {
          i16x4_t h[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int row = 32 * j + 16 * hh + 4 * g + (l16 >> 2);
            const int chunk = 2 * db + ((l16 & 3) >> 1);
            const unsigned char* p = vbuf + row * (DH * 2) + ((chunk ^ (row & kSwV)) * 16) + (l16 & 1) * 8;
            h[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
          }
          const u32x2_t w0 = __builtin_bit_cast(u32x2_t, h[0]);
          const u32x2_t w1 = __builtin_bit_cast(u32x2_t, h[1]);
          v8 = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
        }
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v8, pf, o[db], 0, 0, 0);
      }
    }
  }
#undef DDT_DMA_TILE
  if (!computes) return;

  const float l_tot = rows_sum(l_run);
  if (r >= a.M) return;
  if (it.nsplit == 1) {
    elem* orow = static_cast<elem*>(a.out) + ((static_cast<long>(b) * a.N + node) * a.Hq + head) * DH;
    const bool valid = node < nn;
    const float inv = valid && l_tot > 0.f ? 1.0f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) PolicyBF16<DH>::store_out(orow + db * 16 + 4 * g, o[db] * inv);
    if (a.lse && g == 0)
      a.lse[(static_cast<long>(b) * a.N + node) * a.Hq + head] =
          valid ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_huge_valf();
  } else {
    // bf16 partials: half the round trip of fp32 ones; the combine's result
    // is rounded to bf16 anyway.
    const long pr = (static_cast<long>(sid) * a.Hkv + kvh) * a.M + r;
    uint16_t* dst = static_cast<uint16_t*>(a.ws_o) + pr * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db) PolicyBF16<DH>::store_out(dst + db * 16 + 4 * g, o[db]);
    if (g == 0) a.ws_ml[pr] = make_float2(m_run, l_tot);
  }
}

// ------------------------------------------------------------------ combine
// WPR waves per (request, KV head, query row), 4 / WPR rows per workgroup.
// The waves of a row take its splits w, w + WPR, w + 2·WPR, ...; each issues
// the loads of up to kCombU of them at once (every lane reads the split's
// (max, sum) pair and Dh/64 output dims), so a row with up to WPR·kCombU
// splits costs one round trip to memory.  With WPR = 1 a wave merges its row
// alone; otherwise the row's waves meet in LDS.  The host takes the smallest
// WPR whose round covers the most splits of any request: few splits (large
// batches) get one wave per row, so the grid does not carry four mostly idle
// waves per row.
constexpr int kCombU = 8;

template <typename PT, int PER>
__device__ __forceinline__ void load_partial(const PT* src, float (&v)[PER]) {
  if constexpr (sizeof(PT) == 2) {
    static_assert(PER == 2, "bf16 partials: two dims per lane");
    const uint32_t w = *reinterpret_cast<const uint32_t*>(src);
    v[0] = __uint_as_float(w << 16);
    v[1] = __uint_as_float(w & 0xffff0000u);
  } else {
#pragma unroll
    for (int k = 0; k < PER; ++k) v[k] = src[k];
  }
}

template <typename elem, typename PT, int DH, int WPR>
__global__ __launch_bounds__(256) void combine_kernel(AttnArgs a) {
  constexpr int PER = DH / 64;                // output dims per lane
  constexpr int RPW = 4 / WPR;                // rows per workgroup
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_acc[WPR > 1 ? 4 : 1][DH];
  const int b = blockIdx.x / a.Hkv, kvh = blockIdx.x % a.Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = blockIdx.y * RPW + wave / WPR, sub = wave % WPR;
  int start, ns;
  if (a.tab_n > 0) {
    start = a.tab_split0[b];
    ns = a.tab_split0[b + 1] - start;
    if (a.dyn_len) {
      // the splits the main kernel ran for the length in device memory
      const int Ld = min(max(a.ctx_len[b], 0), a.tab_len[b]);
      ns = min(ns, Ld > 0 ? (Ld + a.split_keys - 1) / a.split_keys : 1);
    }
  } else {
    const int SK = a.split_keys;
    auto nsplits = [&](int bb) {
      int off, L;
      ctx_range(a, bb, &off, &L);
      return L > 0 ? (L + SK - 1) / SK : 1;
    };
    ns = nsplits(b);
    start = 0;
    for (int bb = lane; bb < b; bb += 64) start += nsplits(bb);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) start += __shfl_xor(start, o, 64);
    // the device lengths must match the host copy the grid was planned from;
    // if they do not, never read partials past the planned ones
    if (start >= a.total_splits) return;
    ns = min(ns, a.total_splits - start);
  }
  if (ns <= 1) return;                        // the same for the whole workgroup
  // a row past M (the last workgroup's spare waves) or a padding node does no
  // merge, but its waves still reach the barrier below
  bool live = r < a.M;
  const int node = r / a.G, head = kvh * a.G + r % a.G;
  const long orow = (static_cast<long>(b) * a.N + node) * a.Hq + head;
  elem* dst = static_cast<elem*>(a.out) + orow * DH;
  if (live && node >= a.num_nodes[b]) {
    if (sub == 0) {
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        if constexpr (sizeof(elem) == 2) dst[lane * PER + k] = 0; else dst[lane * PER + k] = 0.f;
      }
      if (a.lse && lane == 0) a.lse[orow] = -__builtin_huge_valf();
    }
    live = false;
  }
  const long pr0 = static_cast<long>(start) * a.Hkv + kvh;
  auto prow = [&](int sp) { return (pr0 + static_cast<long>(sp) * a.Hkv) * a.M + r; };
  const PT* ws = static_cast<const PT*>(a.ws_o);
  float mw = kNegBig, lw = 0.f, acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) acc[k] = 0.f;
  for (int sp0 = sub; live && sp0 < ns; sp0 += WPR * kCombU) {
    float2 ml[kCombU];
    float v[kCombU][PER];
    // unconditional loads (of the last split where there is none, then
    // masked): a load under a condition is waited for on its own, so the
    // conditional form took one round trip per split
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const long pr = prow(min(sp0 + WPR * u, ns - 1));
      ml[u] = a.ws_ml[pr];
      load_partial<PT, PER>(ws + pr * DH + lane * PER, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      if (sp0 + WPR * u >= ns) {
        ml[u] = make_float2(kNegBig, 0.f);
#pragma unroll
        for (int k = 0; k < PER; ++k) v[u][k] = 0.f;
      }
    }
    float mc = mw;
#pragma unroll
    for (int u = 0; u < kCombU; ++u) mc = max(mc, ml[u].x);
    const float fr = __builtin_amdgcn_exp2f(mw - mc);
    lw *= fr;
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] *= fr;
#pragma unroll
    for (int u = 0; u < kCombU; ++u) {
      const float w = __builtin_amdgcn_exp2f(ml[u].x - mc);
      lw += w * ml[u].y;
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] += w * v[u][k];
    }
    mw = mc;
  }
  if constexpr (WPR == 1) {
    if (!live) return;
    const float inv = lw > 0.f ? 1.0f / lw : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const float o = acc[k] * inv;
      if constexpr (sizeof(elem) == 2) dst[lane * PER + k] = f32_to_bf16_rne(o);
      else dst[lane * PER + k] = o;
    }
    if (a.lse && lane == 0) a.lse[orow] = (mw + __log2f(lw)) * kLn2;
  } else {
    if (lane == 0) {
      s_m[wave] = mw;
      s_l[wave] = lw;
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) s_acc[wave][lane * PER + k] = acc[k];
    __syncthreads();
    if (!live || sub != 0) return;
    float mstar = s_m[wave];
#pragma unroll
    for (int w = 1; w < WPR; ++w) mstar = max(mstar, s_m[wave + w]);
    float f[WPR], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < WPR; ++w) {
      f[w] = __builtin_amdgcn_exp2f(s_m[wave + w] - mstar);
      lsum += f[w] * s_l[wave + w];
    }
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int d = lane * PER + k;
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < WPR; ++w) o += f[w] * s_acc[wave + w][d];
      o *= inv;
      if constexpr (sizeof(elem) == 2) dst[d] = f32_to_bf16_rne(o); else dst[d] = o;
    }
    if (a.lse && lane == 0) a.lse[orow] = (mstar + __log2f(lsum)) * kLn2;
  }
}

// ------------------------------------------------------------------ host side
int keys_per_tile(ddtree_dtype dt, int Dh, int /*qb*/) {
  const int ch = Dh * (dt == DDTREE_BF16 ? 2 : 4) / 16;
  return 1024 / ch;
}

// Keys per split: about 512 workgroups over the whole context (two per CU),
// at least 320 keys (five 64-key tiles: each workgroup's prologue latency and
// each partial's combine cost are spread over enough tiles; on an 8192-token
// context 320 measured 6% faster than 256 and 4% faster than 384) and at most
// 2048 (bounds the imbalance of ragged batches); whole tiles.  A tuning
// request (ddtree_tree_attention_tuned) replaces the plan with its own split
// size.
// Host copy of the context ranges: packed offsets [B+1], or per-request
// (start, length) pairs.  Read in place: the host side allocates nothing.
struct HostRanges {
  const int32_t* offs;    // packed form, or null
  const int32_t* start;   // range form
  const int32_t* len;
  int start_of(int b) const { return offs ? offs[b] : start[b]; }
  int len_of(int b) const { return std::max(0, offs ? offs[b + 1] - offs[b] : len[b]); }
};

int plan_split_keys(const HostRanges& hr, int B, int Hkv, int kt, const ddtree_attention_tuning* tu) {
  long total = 0;
  for (int b = 0; b < B; ++b) total += hr.len_of(b);
  constexpr int kTargetWorkgroups = 512;
  long sk = (total * Hkv + kTargetWorkgroups - 1) / kTargetWorkgroups;
  sk = std::min<long>(std::max<long>(sk, 320), 2048);
  sk = std::max<long>(sk, kt);
  sk = (sk + kt - 1) / kt * kt;
  if (tu && tu->split_keys > 0) sk = (static_cast<long>(tu->split_keys) + kt - 1) / kt * kt;
  return static_cast<int>(std::min<long>(sk, 1L << 30));
}

int count_splits(const HostRanges& hr, int B, int sk, bool* any_multi) {
  int tot = 0;
  *any_multi = false;
  for (int b = 0; b < B; ++b) {
    const int L = hr.len_of(b);
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

// LDS ring depth.  Two stages (64 KB) let two workgroups share a CU, each
// with one tile in flight while it computes the other.  Three and four
// stages (4-wave form only) measured no faster, also for grids of at most one
// workgroup per CU, where they would not cost occupancy; a tuning request
// selects them.
template <int QB, int NS>
void launch_dma_qbs(const AttnArgs& a, int total_splits, hipStream_t st) {
  constexpr int NW = QB <= 4 ? 4 : 8;
  const size_t lds = static_cast<size_t>(NS) * 2 * 64 * 128 * 2;
  const dim3 grid(total_splits, a.Hkv, (a.M + 127) / 128);
  hipLaunchKernelGGL((attn_dma_kernel<QB, NW, NS>), grid, dim3(NW * 64), lds, st, a);
}

template <int QB>
void launch_dma_qb(const AttnArgs& a, int total_splits, int stages, hipStream_t st) {
  if constexpr (QB <= 4) {
    switch (stages) {
      case 3: launch_dma_qbs<QB, 3>(a, total_splits, st); return;
      case 4: launch_dma_qbs<QB, 4>(a, total_splits, st); return;
      default: break;
    }
  }
  launch_dma_qbs<QB, 2>(a, total_splits, st);
}

void launch_dma(int qb, const AttnArgs& a, int total_splits, int stages, hipStream_t st) {
  switch (qb) {
    case 1: launch_dma_qb<1>(a, total_splits, stages, st); break;
    case 2: launch_dma_qb<2>(a, total_splits, stages, st); break;
    case 3: launch_dma_qb<3>(a, total_splits, stages, st); break;
    case 4: launch_dma_qb<4>(a, total_splits, stages, st); break;
    case 5: launch_dma_qb<5>(a, total_splits, stages, st); break;
    case 6: launch_dma_qb<6>(a, total_splits, stages, st); break;
    case 7: launch_dma_qb<7>(a, total_splits, stages, st); break;
    default: launch_dma_qb<8>(a, total_splits, stages, st); break;
  }
}

size_t workspace_bytes_for(int B, int N, int Hq, int Hkv, int Dh, const HostRanges& hr,
                           const ddtree_attention_tuning* tu) {
  const int M = N * (Hq / Hkv);
  const int qb = (M + 15) / 16;
  size_t best = 0;
  for (ddtree_dtype dt : {DDTREE_BF16, DDTREE_F32}) {
    const int sk = plan_split_keys(hr, B, Hkv, keys_per_tile(dt, Dh, qb), tu);
    bool multi;
    const int tot = count_splits(hr, B, sk, &multi);
    if (!multi) continue;
    const size_t need = static_cast<size_t>(tot) * Hkv * M * (Dh * sizeof(float) + sizeof(float2));
    best = std::max(best, need);
  }
  return best;
}

ddtree_status attention_impl_args_error(const char* who, int Hq, int Hkv, int Dh) {
  if (Dh != 64 && Dh != 128)
    return fail(DDTREE_EUNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", who, Dh);
  return fail(DDTREE_EINVAL, "%s: Hq=%d must be a multiple of Hkv=%d", who, Hq, Hkv);
}

template <int WPR>
void launch_combine(const AttnArgs& a, ddtree_dtype dtype, int Dh, hipStream_t stream) {
  constexpr int RPW = 4 / WPR;
  const dim3 g(a.B * a.Hkv, (a.M + RPW - 1) / RPW);
  if (dtype == DDTREE_BF16) {
    if (Dh == 128)
      hipLaunchKernelGGL((combine_kernel<uint16_t, uint16_t, 128, WPR>), g, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<uint16_t, float, 64, WPR>), g, dim3(256), 0, stream, a);
  } else {
    if (Dh == 128) hipLaunchKernelGGL((combine_kernel<float, float, 128, WPR>), g, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((combine_kernel<float, float, 64, WPR>), g, dim3(256), 0, stream, a);
  }
}

// Shared body of the packed-offset and range forms.  hr: host copy of the
// context ranges (validated by the caller); a.ctx_offsets or a.ctx_start /
// ctx_len already set to the device arrays.
ddtree_status attention_impl(AttnArgs& a, const char* who, const void* q, const void* k_ctx,
                             const void* v_ctx, const HostRanges& hr,
                             const void* k_tree, const void* v_tree, const ddtree_tree* tree,
                             int32_t Hq, int32_t Hkv, int32_t Dh, ddtree_dtype dtype, float scale,
                             void* out, float* lse, void* workspace, size_t workspace_bytes,
                             const ddtree_attention_tuning* tu, hipStream_t stream) {
  if (!q || !k_tree || !v_tree || !out) return fail(DDTREE_EINVAL, "%s: null pointer", who);
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "%s: unknown dtype %d", who, static_cast<int>(dtype));
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0)
    return fail(DDTREE_EINVAL, "%s: Hq=%d must be a multiple of Hkv=%d", who, Hq, Hkv);
  if (Dh != 64 && Dh != 128)
    return fail(DDTREE_EUNSUPPORTED, "%s: head_dim %d (supported: 64, 128)", who, Dh);
  // scale 0 selects the usual 1/sqrt(Dh)
  if (scale == 0.0f) scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(Dh)));
  if (!(scale > 0.0f) || !(scale < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "%s: scale must be > 0 and finite (or 0 for 1/sqrt(Dh))", who);
  if (tu && (tu->split_keys < 0 || tu->stages < 0 || tu->stages == 1 || tu->stages > 4))
    return fail(DDTREE_EINVAL, "%s: tuning: split_keys %d (>= 0), stages %d (0, 2, 3 or 4)", who,
                tu->split_keys, tu->stages);
  const int B = tree->B, N = tree->N;
  const int M = N * (Hq / Hkv);
  if (M > 1024)
    return fail(DDTREE_EUNSUPPORTED, "%s: %d query rows per KV head (N * Hq / Hkv) exceed 1024",
                who, M);
  long total = 0;
  for (int b = 0; b < B; ++b) total += hr.len_of(b);
  if (total > 0 && (!k_ctx || !v_ctx)) return fail(DDTREE_EINVAL, "%s: null context K/V", who);
  if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out) ||
      (k_ctx && !aligned16(k_ctx)) || (v_ctx && !aligned16(v_ctx)))
    return fail(DDTREE_EINVAL, "%s: tensors must be 16-byte aligned", who);
  const int qb = (std::min(M, 128) + 15) / 16;   // 16-row query blocks per slice
  const int kt = keys_per_tile(dtype, Dh, qb);
  const int sk = plan_split_keys(hr, B, Hkv, kt, tu);
  bool multi;
  const int splits = count_splits(hr, B, sk, &multi);
  a.q = q;
  a.k_ctx = k_ctx;
  a.v_ctx = v_ctx;
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
  a.total_splits = splits;
  a.tab_n = 0;
  if (a.dyn_len && B > kTabMax)
    return fail(DDTREE_EUNSUPPORTED, "%s: more than %d requests", who, kTabMax);
  if (B <= kTabMax) {
    a.tab_n = B;
    int acc = 0;
    for (int b = 0; b < B; ++b) {
      a.tab_split0[b] = acc;
      a.tab_off[b] = hr.start_of(b);
      a.tab_len[b] = hr.len_of(b);
      acc += a.tab_len[b] > 0 ? (a.tab_len[b] + sk - 1) / sk : 1;
    }
    a.tab_split0[B] = acc;
  }
  a.out = out;
  a.lse = lse;
  a.ws_o = nullptr;
  a.ws_ml = nullptr;
  if (multi) {
    const size_t need = static_cast<size_t>(splits) * Hkv * M * Dh * sizeof(float);
    const size_t need_ml = static_cast<size_t>(splits) * Hkv * M * sizeof(float2);
    if (!workspace || workspace_bytes < need + need_ml || !aligned16(workspace))
      return fail(DDTREE_EINVAL, "%s: workspace of %zu bytes needed, got %zu", who,
                  need + need_ml, workspace_bytes);
    a.ws_o = workspace;
    a.ws_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + need);
  }
  if (dtype == DDTREE_BF16) {
    if (Dh == 128) launch_dma(qb, a, splits, tu && tu->stages > 0 ? tu->stages : 2, stream);
    else launch_qb<PolicyBF16<64>>(qb, a, splits, stream);
  } else {
    if (Dh == 128) launch_qb<PolicyF32<128>>(qb, a, splits, stream);
    else launch_qb<PolicyF32<64>>(qb, a, splits, stream);
  }
  if (multi) {
    int max_ns = 1;
    for (int b = 0; b < B; ++b) {
      const long L = hr.len_of(b);
      max_ns = std::max<long>(max_ns, L > 0 ? (L + sk - 1) / sk : 1);
    }
    const int wpr = max_ns <= kCombU ? 1 : max_ns <= 2 * kCombU ? 2 : 4;
    if (wpr == 1) launch_combine<1>(a, dtype, Dh, stream);
    else if (wpr == 2) launch_combine<2>(a, dtype, Dh, stream);
    else launch_combine<4>(a, dtype, Dh, stream);
  }
  return check_launch(who);
}

// The device address of `scratch` on the current device, looked up once per
// device with that device current (each GPU has its own copy of the array).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

ddtree_status scratch_address(void** out, const char* who) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(DDTREE_EDEVICE, "%s: no current device (or device %d beyond %d)", who, dev,
                kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DDTREE_EDEVICE, "%s: hipGetSymbolAddress of the scratch array: %s", who,
                  hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DDTREE_OK;
}

// Validation and launch of the packed-offset form (planned, tuned or no-allocation).
ddtree_status packed_attention(const char* who, const void* q, const void* k_ctx,
                               const void* v_ctx, const int32_t* ctx_offsets,
                               const int32_t* ctx_offsets_host, const void* k_tree,
                               const void* v_tree, const ddtree_tree* tree, int32_t Hq,
                               int32_t Hkv, int32_t Dh, ddtree_dtype dtype, float scale, void* out,
                               float* lse, void* workspace, size_t workspace_bytes,
                               const ddtree_attention_tuning* tuning, bool use_scratch,
                               hipStream_t stream) {
  ddtree_status st = check_tree(tree, who);
  if (st != DDTREE_OK) return st;
  if (!ctx_offsets || !ctx_offsets_host) return fail(DDTREE_EINVAL, "%s: null pointer", who);
  const int B = tree->B;
  if (ctx_offsets_host[0] != 0) return fail(DDTREE_EINVAL, "%s: ctx_offsets[0] must be 0", who);
  for (int b = 0; b < B; ++b)
    if (ctx_offsets_host[b + 1] < ctx_offsets_host[b])
      return fail(DDTREE_EINVAL, "%s: ctx_offsets must be non-decreasing", who);
  const HostRanges hr{ctx_offsets_host, nullptr, nullptr};
  if (use_scratch) {
    if (Hkv < 1 || Hq % Hkv != 0 || (Dh != 64 && Dh != 128))
      return attention_impl_args_error(who, Hq, Hkv, Dh);
    const size_t need = workspace_bytes_for(B, tree->N, Hq, Hkv, Dh, hr, nullptr);
    if (need > DDTREE_NOALLOC_SCRATCH_BYTES)
      return fail(DDTREE_EUNSUPPORTED,
                  "%s: the split partials need %zu bytes, more than the %zu bytes of its device "
                  "scratch (use ddtree_tree_attention with a workspace)",
                  who, need, static_cast<size_t>(DDTREE_NOALLOC_SCRATCH_BYTES));
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      st = scratch_address(&workspace, who);
      if (st != DDTREE_OK) return st;
      workspace_bytes = DDTREE_NOALLOC_SCRATCH_BYTES;
    }
  }
  AttnArgs a;
  a.ctx_offsets = ctx_offsets;
  a.ctx_start = nullptr;
  a.ctx_len = nullptr;
  a.dyn_len = 0;
  return attention_impl(a, who, q, k_ctx, v_ctx, hr, k_tree, v_tree, tree, Hq, Hkv, Dh, dtype,
                        scale, out, lse, workspace, workspace_bytes, tuning, stream);
}

}  // namespace
}  // namespace ddt

extern "C" size_t ddtree_tree_attention_tuned_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                                             int32_t Hkv, int32_t Dh,
                                                             const int32_t* ctx_offsets_host,
                                                             const ddtree_attention_tuning* tuning) {
  using namespace ddt;
  if (B < 1 || N < 1 || Hkv < 1 || Hq % Hkv != 0 || !ctx_offsets_host || (Dh != 64 && Dh != 128))
    return 0;
  return workspace_bytes_for(B, N, Hq, Hkv, Dh, HostRanges{ctx_offsets_host, nullptr, nullptr},
                             tuning);
}

extern "C" size_t ddtree_tree_attention_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                                       int32_t Hkv, int32_t Dh,
                                                       const int32_t* ctx_offsets_host) {
  return ddtree_tree_attention_tuned_workspace_size(B, N, Hq, Hkv, Dh, ctx_offsets_host, nullptr);
}

extern "C" size_t ddtree_tree_attention_ranges_workspace_size(int32_t B, int32_t N, int32_t Hq,
                                                              int32_t Hkv, int32_t Dh,
                                                              const int32_t* ctx_len_host) {
  using namespace ddt;
  if (B < 1 || N < 1 || Hkv < 1 || Hq % Hkv != 0 || !ctx_len_host || (Dh != 64 && Dh != 128))
    return 0;
  return workspace_bytes_for(B, N, Hq, Hkv, Dh, HostRanges{nullptr, ctx_len_host, ctx_len_host},
                             nullptr);
}

extern "C" ddtree_status ddtree_tree_attention_tuned(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_offsets,
    const int32_t* ctx_offsets_host, const void* k_tree, const void* v_tree,
    const ddtree_tree* tree, int32_t Hq, int32_t Hkv, int32_t Dh, ddtree_dtype dtype,
    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
    const ddtree_attention_tuning* tuning, hipStream_t stream) {
  return ddt::packed_attention(tuning ? "ddtree_tree_attention_tuned" : "ddtree_tree_attention",
                               q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree, v_tree,
                               tree, Hq, Hkv, Dh, dtype, scale, out, lse, workspace,
                               workspace_bytes, tuning, false, stream);
}

extern "C" ddtree_status ddtree_tree_attention_noalloc(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_offsets,
    const int32_t* ctx_offsets_host, const void* k_tree, const void* v_tree,
    const ddtree_tree* tree, int32_t Hq, int32_t Hkv, int32_t Dh, ddtree_dtype dtype,
    float scale, void* out, float* lse, hipStream_t stream) {
  return ddt::packed_attention("ddtree_tree_attention_noalloc", q, k_ctx, v_ctx, ctx_offsets,
                               ctx_offsets_host, k_tree, v_tree, tree, Hq, Hkv, Dh, dtype, scale,
                               out, lse, nullptr, 0, nullptr, true, stream);
}

extern "C" ddtree_status ddtree_tree_attention(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_offsets,
    const int32_t* ctx_offsets_host, const void* k_tree, const void* v_tree,
    const ddtree_tree* tree, int32_t Hq, int32_t Hkv, int32_t Dh, ddtree_dtype dtype,
    float scale, void* out, float* lse, void* workspace, size_t workspace_bytes,
    hipStream_t stream) {
  return ddtree_tree_attention_tuned(q, k_ctx, v_ctx, ctx_offsets, ctx_offsets_host, k_tree,
                                     v_tree, tree, Hq, Hkv, Dh, dtype, scale, out, lse, workspace,
                                     workspace_bytes, nullptr, stream);
}

namespace ddt {
namespace {

// Validation and launch of the range forms: exact lengths (capped = false)
// or upper bounds of lengths read from the device when the kernels run.
ddtree_status ranges_attention(const char* who, bool capped, const void* q, const void* k_ctx,
                               const void* v_ctx, const int32_t* ctx_start,
                               const int32_t* ctx_len, const int32_t* ctx_start_host,
                               const int32_t* ctx_len_host, const void* k_tree,
                               const void* v_tree, const ddtree_tree* tree, int32_t Hq,
                               int32_t Hkv, int32_t Dh, ddtree_dtype dtype, float scale,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  ddtree_status st = check_tree(tree, who);
  if (st != DDTREE_OK) return st;
  if (!ctx_start || !ctx_len || !ctx_start_host || !ctx_len_host)
    return fail(DDTREE_EINVAL, "%s: null pointer", who);
  for (int b = 0; b < tree->B; ++b)
    if (ctx_start_host[b] < 0 || ctx_len_host[b] < 0 ||
        static_cast<long>(ctx_start_host[b]) + ctx_len_host[b] > INT32_MAX)
      return fail(DDTREE_EINVAL, "%s: request %d: context start %d, length %d", who, b,
                  ctx_start_host[b], ctx_len_host[b]);
  AttnArgs a;
  a.ctx_offsets = nullptr;
  a.ctx_start = ctx_start;
  a.ctx_len = ctx_len;
  a.dyn_len = capped ? 1 : 0;
  return attention_impl(a, who, q, k_ctx, v_ctx, HostRanges{nullptr, ctx_start_host, ctx_len_host},
                        k_tree, v_tree, tree, Hq, Hkv, Dh, dtype, scale, out, lse, workspace,
                        workspace_bytes, nullptr, stream);
}

}  // namespace
}  // namespace ddt

extern "C" ddtree_status ddtree_tree_attention_ranges(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_start,
    const int32_t* ctx_len, const int32_t* ctx_start_host, const int32_t* ctx_len_host,
    const void* k_tree, const void* v_tree, const ddtree_tree* tree, int32_t Hq, int32_t Hkv,
    int32_t Dh, ddtree_dtype dtype, float scale, void* out, float* lse, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  return ddt::ranges_attention("ddtree_tree_attention_ranges", false, q, k_ctx, v_ctx, ctx_start,
                               ctx_len, ctx_start_host, ctx_len_host, k_tree, v_tree, tree, Hq,
                               Hkv, Dh, dtype, scale, out, lse, workspace, workspace_bytes,
                               stream);
}

extern "C" ddtree_status ddtree_tree_attention_ranges_capped(
    const void* q, const void* k_ctx, const void* v_ctx, const int32_t* ctx_start,
    const int32_t* ctx_len, const int32_t* ctx_start_host, const int32_t* ctx_cap_host,
    const void* k_tree, const void* v_tree, const ddtree_tree* tree, int32_t Hq, int32_t Hkv,
    int32_t Dh, ddtree_dtype dtype, float scale, void* out, float* lse, void* workspace,
    size_t workspace_bytes, hipStream_t stream) {
  return ddt::ranges_attention("ddtree_tree_attention_ranges_capped", true, q, k_ctx, v_ctx,
                               ctx_start, ctx_len, ctx_start_host, ctx_cap_host, k_tree, v_tree,
                               tree, Hq, Hkv, Dh, dtype, scale, out, lse, workspace,
                               workspace_bytes, stream);
}
