// ddtree_vocab_top_p: the top-p nucleus of every node's integer target law.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
// Evaluation Strategy", Section 3: top_p is threaded through to the verify
// walk, which then samples from the truncated, renormalised target row.  The
// nucleus is the shortest prefix of the row's tokens ordered by (weight desc,
// id asc) whose weight sum S reaches p of the total, decided exactly as
// 2^32 * S >= P * R with P = rint(p * 2^32).  It is described by its last
// token: threshold weight w* and id*; a token is kept iff w > w*, or w = w*
// and id <= id*.
//
// One 512-thread workgroup per node row, up to three per CU (50 KB of LDS
// and at most 80 registers each), so that more loads are in flight per CU.
// With Tt = ceil(P * R / 2^32):
//  1. a pass over the row sums and counts the weights at or above 2^e and
//     copies those tokens (weight, id) to LDS, each wave into its own region
//     (positions from a ballot and a wave-uniform count: no atomics); it
//     succeeds when the sum reaches Tt and every wave's tokens fit its region
//     (kTpCap in all), and the regions are then packed into one list; e
//     starts at 20 and is moved by bisection between exponents known to reach
//     Tt and not to (1-4 passes);
//  2. candidates in LDS: the workgroup sorts them by (weight desc, id asc)
//     and scans their weights in that order; the nucleus's last token is the
//     one whose running sum first reaches Tt, which gives w*, id* and R_p at
//     once (steps 4-5 below describe the same cut);
//     more than kTpCap tokens needed: w* = the largest v with
//     sum{w >= v} >= Tt, by 8-way interval search (7 thresholds per
//     reduction) over the row itself (exact, slower);
//  3. every pass over the row skips the weight polynomial of the tokens that
//     provably weigh less than the pass's lower bound;
//  4. with S> = sum{w > w*}, the nucleus takes m = ceil((Tt - S>) / w*) of the
//     tokens of weight w*, the smallest ids: id* = the smallest X with
//     #{w = w*, id <= X} >= m, by the same search over ids;
//  5. R_p = S> + m * w*, and the kept weights are summed per DDTREE_R_BLOCK
//     tokens for the walk's residual draw.
#include "common.hpp"

namespace ddt {
namespace {

constexpr int kTpThreads = 512;
constexpr int kTpWaves = kTpThreads / kWave;
constexpr int kTpCap = 4096;       // candidate tokens held in LDS (12 bytes each)
constexpr int kTpRegion = kTpCap / (kTpThreads / kWave);   // per-wave share during a pass
constexpr int kTpProbes = 7;       // thresholds per search round (8-way search)
constexpr int kMaxSums = 8;       // sums per block-wide reduction (and slot rows of the sorted cut)

struct TpShared {
  uint64_t w[kTpCap];
  uint32_t id[kTpCap];
  uint64_t part[kTpWaves][kMaxSums];
  uint64_t tot[kMaxSums];
  uint64_t blk[kWave];
  int cnt[kTpThreads / kWave];
};

// Sums of K per-thread values over the workgroup; every thread gets the totals.
template <int K>
__device__ __forceinline__ void block_sums(uint64_t (&v)[K], TpShared& s, int tid) {
  static_assert(K <= kMaxSums, "partial-sum buffer too small");
  const int lane = tid & (kWave - 1), wave = tid / kWave;
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum_u64_dpp(v[k]);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) s.part[wave][k] = v[k];
  }
  __syncthreads();
  if (tid < K) {
    uint64_t a = 0;
    for (int w = 0; w < kTpWaves; ++w) a += s.part[w][tid];
    s.tot[tid] = a;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = s.tot[k];
}

// Lane l's copy of lane l ^ j's 64-bit value (j < 64, a power of two): DPP for
// the in-row distances 1, 2 and 8, a bpermute through LDS for the others.
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int j, int lane) {
  int lo = static_cast<int>(static_cast<uint32_t>(v)), hi = static_cast<int>(static_cast<uint32_t>(v >> 32));
  if (j == 1) {
    lo = __builtin_amdgcn_mov_dpp(lo, 0xB1, 0xF, 0xF, false);   // quad_perm [1, 0, 3, 2]
    hi = __builtin_amdgcn_mov_dpp(hi, 0xB1, 0xF, 0xF, false);
  } else if (j == 2) {
    lo = __builtin_amdgcn_mov_dpp(lo, 0x4E, 0xF, 0xF, false);   // quad_perm [2, 3, 0, 1]
    hi = __builtin_amdgcn_mov_dpp(hi, 0x4E, 0xF, 0xF, false);
  } else if (j == 8) {
    lo = __builtin_amdgcn_mov_dpp(lo, 0x128, 0xF, 0xF, false);  // row_ror 8: l + 8 mod 16 = l ^ 8
    hi = __builtin_amdgcn_mov_dpp(hi, 0x128, 0xF, 0xF, false);
  } else {
    const int addr = (lane ^ j) << 2;
    lo = __builtin_amdgcn_ds_bpermute(addr, lo);
    hi = __builtin_amdgcn_ds_bpermute(addr, hi);
  }
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

constexpr int kTpKeyIdBits = 22;   // ids < V <= 64 * DDTREE_R_BLOCK = 2^21
constexpr uint64_t kTpKeyIdMask = (1ull << kTpKeyIdBits) - 1;

// The nucleus of a candidate list of at most E * kTpThreads tokens, by the
// whole workgroup: every candidate becomes the key (w << 22) | (2^22 - 1 - id),
// unique per token and larger for a token earlier in the (weight desc, id asc)
// order; a bitonic network sorts the keys descending over E * kTpThreads slots
// (slot g = e * kTpThreads + tid; empty slots hold key 0, below every
// candidate, since a candidate weighs at least 1); an inclusive scan of the
// weights in that order then gives each token the mass up to and including it,
// and the nucleus is every token whose mass before it is below Tt, its last
// token the one whose scan first reaches Tt.  Exact integer arithmetic: the
// same cut as the interval searches below.
template <int E>
__device__ void nucleus_by_sort(TpShared& s, int nc, int tid, uint64_t Tt, long row, int nb,
                                uint64_t* __restrict__ thr_w, int32_t* __restrict__ thr_id,
                                uint64_t* __restrict__ Rp, uint64_t* __restrict__ Rp_blocks) {
  constexpr int n = E * kTpThreads;
  static_assert(n <= kTpCap && E <= kMaxSums, "the exchange buffers live in the candidate list");
  constexpr bool kTwoBuffers = 2 * n <= kTpCap;
  const int lane = tid & (kWave - 1), wave = tid / kWave;
  uint64_t k[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int g = e * kTpThreads + tid;
    k[e] = g < nc ? (s.w[g] << kTpKeyIdBits) | (kTpKeyIdMask - s.id[g]) : 0ull;
  }
  if (tid < kWave) s.blk[tid] = 0;
  __syncthreads();   // the candidate list is read: its space holds the exchanges now
  int parity = 0;
#pragma unroll
  for (int kk = 2; kk <= n; kk <<= 1) {
#pragma unroll
    for (int j = kk >> 1; j > 0; j >>= 1) {
      if (j >= kTpThreads) {
        // the partner slot is one of this thread's own; bit kk of the lower
        // slot (the same for every thread) gives the run's direction
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e * kTpThreads) & j) continue;
          const int e2 = e + j / kTpThreads;
          const bool desc = ((e * kTpThreads) & kk) == 0;
          const uint64_t a = k[e], b = k[e2];
          const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
          k[e] = desc ? hi : lo;
          k[e2] = desc ? lo : hi;
        }
        continue;
      }
      uint64_t o[E];
      if (j >= kWave) {
        // across waves through LDS: with room for two buffers they alternate,
        // so one barrier per step (a buffer is written again only after the
        // next step's barrier, which every thread reaches after its reads of
        // it); with room for one, a second barrier ends the step's reads
        uint64_t* buf = s.w + (kTwoBuffers ? parity * n : 0);
        parity ^= 1;
#pragma unroll
        for (int e = 0; e < E; ++e) buf[e * kTpThreads + tid] = k[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = buf[(e * kTpThreads + tid) ^ j];
        if (!kTwoBuffers) __syncthreads();
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = xor_lane_u64(k[e], j, lane);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int g = e * kTpThreads + tid;
        // descending runs where bit kk of the slot is clear; the lower slot of
        // a pair keeps the larger key in a descending run
        const bool keep_max = ((g & j) == 0) == ((g & kk) == 0);
        k[e] = keep_max ? (k[e] > o[e] ? k[e] : o[e]) : (k[e] < o[e] ? k[e] : o[e]);
      }
    }
  }
  // inclusive scan of the weights in slot order: within the wave by lane
  // moves, then the earlier waves' and earlier slot rows' totals
  uint64_t w[E], incl[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w[e] = k[e] >> kTpKeyIdBits;
    uint64_t v = w[e];
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int src = lane >= d ? lane - d : lane;
      const int lo = __builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(static_cast<uint32_t>(v)));
      const int hi = __builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(static_cast<uint32_t>(v >> 32)));
      if (lane >= d) v += (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
    }
    incl[e] = v;
    if (lane == kWave - 1) s.part[wave][e] = v;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) {
    uint64_t before = 0;
    for (int e2 = 0; e2 < e; ++e2)
      for (int wv = 0; wv < kTpWaves; ++wv) before += s.part[wv][e2];
    for (int wv = 0; wv < wave; ++wv) before += s.part[wv][e];
    incl[e] += before;
    const uint64_t excl = incl[e] - w[e];
    if (w[e] != 0 && excl < Tt) {
      const int id = static_cast<int>(kTpKeyIdMask - (k[e] & kTpKeyIdMask));
      atomicAdd(reinterpret_cast<unsigned long long*>(&s.blk[id / DDTREE_R_BLOCK]),
                static_cast<unsigned long long>(w[e]));
      if (incl[e] >= Tt) {   // the nucleus's last token: exactly one slot
        thr_w[row] = w[e];
        thr_id[row] = id;
        Rp[row] = incl[e];
      }
    }
  }
  __syncthreads();
  if (tid < nb) Rp_blocks[row * nb + tid] = s.blk[tid];
}

template <typename T>
__global__ __launch_bounds__(kTpThreads, 6) void top_p_kernel(
    const T* __restrict__ logits, int N, int V, const int32_t* __restrict__ num_nodes,
    const float* __restrict__ maxv, const uint64_t* __restrict__ R, WeightConsts wc, uint64_t P,
    uint64_t* __restrict__ thr_w, int32_t* __restrict__ thr_id, uint64_t* __restrict__ Rp,
    uint64_t* __restrict__ Rp_blocks) {
  __shared__ TpShared s;
  const int n = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const long row = static_cast<long>(b) * N + n;
  const int nb = (V + DDTREE_R_BLOCK - 1) / DDTREE_R_BLOCK;   // <= 64 (checked on the host)
  if (n >= num_nodes[b]) {
    if (tid == 0) {
      thr_w[row] = 0;
      thr_id[row] = -1;
      Rp[row] = 0;
    }
    if (tid < nb) Rp_blocks[row * nb + tid] = 0;
    return;
  }
  const T* x = logits + row * static_cast<long>(V);
  const float m = maxv[row];
  const uint64_t Rt = R[row];
  // Tt = ceil(P * R / 2^32) exactly: P <= 2^32 and R < 2^51
  const uint64_t Tt = P * (Rt >> 32) + ((P * (Rt & 0xFFFFFFFFull) + 0xFFFFFFFFull) >> 32);
  const int lane = tid & (kWave - 1);

  // f(w, id) for every token of the row (uniformly across the wave: tokens
  // past V come as w = 0), reading 16-byte chunks, four per thread in flight;
  // the weight polynomial runs only for tokens with y = (l - m) * c >= ymin
  // (the others get w = 0)
  constexpr int kVec = 16 / static_cast<int>(sizeof(T));
  const int nchunk = (V + kVec - 1) / kVec;
  const bool vec_ok = aligned16(x);
  auto row_scan = [&](float ymin, auto&& f) {
    for (int c0 = 0; c0 < nchunk; c0 += 4 * kTpThreads) {
      float v[4][kVec];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const long ch = c0 + u * kTpThreads + tid;
        if (vec_ok && (ch + 1) * kVec <= V) {
          const uint4 q = *reinterpret_cast<const uint4*>(x + ch * kVec);
          const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
          for (int k = 0; k < kVec; ++k) {
            if (kVec == 8)
              v[u][k] = __uint_as_float((k & 1) ? (qw[k >> 1] & 0xFFFF0000u) : (qw[k >> 1] << 16));
            else
              v[u][k] = __uint_as_float(qw[k]);
          }
        } else {
#pragma unroll
          for (int k = 0; k < kVec; ++k)
            v[u][k] = ch * kVec + k < V ? Elem<T>::get(x, ch * kVec + k) : -__builtin_huge_valf();
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int id = static_cast<int>((c0 + u * kTpThreads + tid) * kVec + k);
          float y0;
          {
#pragma clang fp contract(off)
            y0 = (v[u][k] - m) * wc.c;
          }
          uint64_t w = 0;
          if (y0 >= ymin) w = weight(v[u][k], m, wc);
          f(w, id);
        }
      }
    }
  };

  // 1. candidates: one pass per attempt sums and counts the weights >= 2^e and
  // copies those tokens to LDS (any order); the attempt succeeds when their sum
  // reaches Tt and they fit.  e starts at 20 and moves by halving the interval
  // between the largest exponent known to reach Tt and the smallest known not to.
  const int wave = tid / kWave;
  int e = 20, e_good = -1, e_bad = 34;
  bool in_lds = false;
  int nc = 0;
  for (int attempt = 0; attempt < 12; ++attempt) {
    const uint64_t lb = 1ull << e;
    const float ymin = static_cast<float>(e - 33);
    uint64_t sc[3] = {0, 0, 0};
    int wcount = 0;   // this wave's tokens so far (the same in every lane)
    auto take = [&](uint64_t w, int id) {
      const bool c = w >= lb;
      if (c) {
        sc[0] += w;
        sc[1] += 1;
      }
      const uint64_t mask = __ballot(c);
      if (mask == 0) return;
      const int pos = wcount + __popcll(mask & ((1ull << lane) - 1ull));
      if (c && pos < kTpRegion) {
        s.w[wave * kTpRegion + pos] = w;
        s.id[wave * kTpRegion + pos] = static_cast<uint32_t>(id);
      }
      wcount += __popcll(mask);
    };
    row_scan(ymin, take);
    if (lane == 0) s.cnt[wave] = wcount;
    sc[2] = wcount > kTpRegion ? 1u : 0u;   // 1 in each lane of a wave whose tokens overflowed
    block_sums<3>(sc, s, tid);
    if (sc[0] >= Tt) {
      e_good = e;
      if (sc[2] == 0) {
        // pack the regions into one list: every thread reads its entries,
        // then (after the barrier) writes them at its region's offset
        constexpr int kPer = kTpCap / kTpThreads;
        constexpr int kRR = kTpThreads / kTpRegion;   // regions per row of entries
        static_assert(kRR * kTpRegion == kTpThreads && kRR <= 2, "entry j of a thread lies in region kRR * j + tid / kTpRegion");
        int pre[kTpThreads / kWave];   // region offsets in the packed list
        int acc = 0;
#pragma unroll
        for (int w = 0; w < kTpThreads / kWave; ++w) {
          pre[w] = acc;
          acc += s.cnt[w];
        }
        const bool upper = kRR == 2 && tid >= kTpRegion;
        const int re = tid - (upper ? kTpRegion : 0);   // entry within its region
        uint64_t pw[kPer];
        uint32_t pid[kPer];
        int dst[kPer];
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int src = j * kTpThreads + tid;
          const int cnt = upper ? s.cnt[kRR * j + 1] : s.cnt[kRR * j];
          const int base = upper ? pre[kRR * j + 1] : pre[kRR * j];
          dst[j] = re < cnt ? base + re : -1;
          pw[j] = s.w[src];
          pid[j] = s.id[src];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          if (dst[j] >= 0) {
            s.w[dst[j]] = pw[j];
            s.id[dst[j]] = pid[j];
          }
        }
        __syncthreads();
        in_lds = true;
        nc = static_cast<int>(sc[1]);
        break;
      }
    } else {
      e_bad = e;
    }
    if (e_good < 0) e = max(0, e - 8);          // 2^0 always reaches Tt (it sums to R)
    else if (e_bad - e_good <= 1) break;         // too many tokens: search the row itself
    else e = (e_good + e_bad) / 2;
  }

  // 2-5. more candidates than the LDS holds: the search by the whole workgroup
  // over the row (workgroup sums)
  auto search = [&](auto&& each, auto&& reduce, auto&& sync, int lid) {
    // invariant: sum{w >= lo} >= Tt > sum{w >= hi}
    uint64_t lo = 1ull << e_good;
    uint64_t hi = 1ull << min(e_bad, 33);
    // 2. w* = the largest v with sum{w >= v} >= Tt: 8-way interval search
    for (int round = 0; round < 40 && hi - lo > 1; ++round) {
      uint64_t th[kTpProbes], acc[kTpProbes];
#pragma unroll
      for (int k = 0; k < kTpProbes; ++k) {
        th[k] = lo + (hi - lo) * static_cast<uint64_t>(k + 1) / (kTpProbes + 1);
        acc[k] = 0;
      }
      each(lo, [&](uint64_t w, int) {
#pragma unroll
        for (int k = 0; k < kTpProbes; ++k) acc[k] += w >= th[k] ? w : 0;
      });
      reduce(acc);
      uint64_t nlo = lo, nhi = hi;
#pragma unroll
      for (int k = 0; k < kTpProbes; ++k) {
        if (acc[k] >= Tt) nlo = max(nlo, th[k]);
        else nhi = min(nhi, th[k]);
      }
      lo = nlo;
      hi = nhi;
    }
    const uint64_t ws = lo;
    // 3. tokens of weight w* that the nucleus takes, and the id cut among them
    uint64_t g[kTpProbes] = {};
    each(ws, [&](uint64_t w, int id) {
      g[0] += w > ws ? w : 0;
      g[1] += w == ws ? 1 : 0;
    });
    reduce(g);
    const uint64_t sgt = g[0];
    const uint64_t take = (Tt - sgt + ws - 1) / ws;   // 1 <= take <= #{w = w*}
    long ilo = -1, ihi = V - 1;                        // #{.. id <= ilo} < take <= #{.. id <= ihi}
    for (int round = 0; round < 40 && ihi - ilo > 1; ++round) {
      long th[kTpProbes];
      uint64_t acc[kTpProbes];
#pragma unroll
      for (int k = 0; k < kTpProbes; ++k) {
        th[k] = ilo + (ihi - ilo) * (k + 1) / (kTpProbes + 1);
        acc[k] = 0;
      }
      each(ws, [&](uint64_t w, int id) {
#pragma unroll
        for (int k = 0; k < kTpProbes; ++k) acc[k] += (w == ws && id <= th[k]) ? 1 : 0;
      });
      reduce(acc);
      long nlo = ilo, nhi = ihi;
#pragma unroll
      for (int k = 0; k < kTpProbes; ++k) {
        if (acc[k] >= take) nhi = min(nhi, th[k]);
        else nlo = max(nlo, th[k]);
      }
      ilo = nlo;
      ihi = nhi;
    }
    const int id_cut = static_cast<int>(ihi);
    // 4. totals: R_p and the kept weight of every token block
    if (lid < kWave) s.blk[lid] = 0;
    sync();
    each(ws, [&](uint64_t w, int id) {
      if (w > ws || (w == ws && id <= id_cut))
        atomicAdd(reinterpret_cast<unsigned long long*>(&s.blk[id / DDTREE_R_BLOCK]),
                  static_cast<unsigned long long>(w));
    });
    sync();
    if (lid == 0) {
      thr_w[row] = ws;
      thr_id[row] = id_cut;
      Rp[row] = sgt + take * ws;
    }
    if (lid < nb) Rp_blocks[row * nb + lid] = s.blk[lid];
  };

  if (in_lds && nc <= kTpThreads) {
    nucleus_by_sort<1>(s, nc, tid, Tt, row, nb, thr_w, thr_id, Rp, Rp_blocks);
  } else if (in_lds && nc <= 2 * kTpThreads) {
    nucleus_by_sort<2>(s, nc, tid, Tt, row, nb, thr_w, thr_id, Rp, Rp_blocks);
  } else if (in_lds && nc <= 4 * kTpThreads) {
    nucleus_by_sort<4>(s, nc, tid, Tt, row, nb, thr_w, thr_id, Rp, Rp_blocks);
  } else if (in_lds) {
    nucleus_by_sort<8>(s, nc, tid, Tt, row, nb, thr_w, thr_id, Rp, Rp_blocks);
  } else {
    search(
        [&](uint64_t bound, auto&& f) {
          // tokens with y below floor(log2 bound) - 33 weigh less than bound / 2
          // (w < 2^(32 + y) * (1 + 1e-6)): they come as w = 0, which no probe counts
          row_scan(static_cast<float>(63 - __builtin_clzll(bound) - 33), f);
        },
        [&](auto& acc) { block_sums<kTpProbes>(acc, s, tid); },
        [&]() { __syncthreads(); }, tid);
  }
}

}  // namespace
}  // namespace ddt

extern "C" ddtree_status ddtree_vocab_top_p(const void* logits, ddtree_dtype dtype, int32_t B,
                                            int32_t N, int32_t V, const int32_t* num_nodes,
                                            const float* maxv, const uint64_t* R,
                                            float temperature, float top_p, uint64_t* thr_w,
                                            int32_t* thr_id, uint64_t* Rp, uint64_t* Rp_blocks,
                                            hipStream_t stream) {
  using namespace ddt;
  const char* who = "ddtree_vocab_top_p";
  if (!logits || !num_nodes || !maxv || !R || !thr_w || !thr_id || !Rp || !Rp_blocks)
    return fail(DDTREE_EINVAL, "%s: null pointer", who);
  if (B < 1 || N < 1 || V < 1 || B > 65535 || N > DDTREE_MAX_NODES)
    return fail(DDTREE_EINVAL, "%s: sizes B=%d N=%d V=%d", who, B, N, V);
  if (V > kWave * DDTREE_R_BLOCK)
    return fail(DDTREE_EUNSUPPORTED, "%s: V = %d exceeds %d", who, V, kWave * DDTREE_R_BLOCK);
  if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf()))
    return fail(DDTREE_EINVAL, "%s: temperature must be > 0 and finite", who);
  if (!(top_p > 0.0f) || !(top_p <= 1.0f))
    return fail(DDTREE_EINVAL, "%s: top_p must be in (0, 1]", who);
  double pd = __builtin_rint(static_cast<double>(top_p) * 4294967296.0);
  if (pd < 1.0) pd = 1.0;
  if (pd > 4294967296.0) pd = 4294967296.0;
  const uint64_t P = static_cast<uint64_t>(pd);
  const WeightConsts wc = weight_consts(temperature);
  const dim3 grid(N, B);
  if (dtype == DDTREE_BF16) {
    hipLaunchKernelGGL(top_p_kernel<uint16_t>, grid, dim3(kTpThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), N, V, num_nodes, maxv, R, wc, P,
                       thr_w, thr_id, Rp, Rp_blocks);
  } else if (dtype == DDTREE_F32) {
    hipLaunchKernelGGL(top_p_kernel<float>, grid, dim3(kTpThreads), 0, stream,
                       static_cast<const float*>(logits), N, V, num_nodes, maxv, R, wc, P, thr_w,
                       thr_id, Rp, Rp_blocks);
  } else {
    return fail(DDTREE_EINVAL, "%s: unknown dtype %d", who, static_cast<int>(dtype));
  }
  return check_launch(who);
}
