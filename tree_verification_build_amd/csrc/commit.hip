// ddtree_commit: the accepted path's tree K/V rows go to the context cache.
//
// "The Architecture of Speculative Decoding: Dissecting DDTree's Tree-Parallel
// Evaluation Strategy", Section 1 step 5 and its summary (the single longest
// verified path is committed) and Section 2 (the cache grows by the committed
// tokens; later steps read it once).  The root and the accepted nodes are
// stored at their tree positions (prefix_len + depth); the next step starts at
// prefix_len + accept_len + 1 with the bonus token as its root.
//
// One workgroup per (request b, path slot j): slot j <= accept_len copies the
// K and V rows ([Hkv, Dh], contiguous in both the tree and the cache layout)
// of path node j with 16-byte loads and stores.  The work is a few KB per
// request: the call is bound by launch and memory latency, not bandwidth.
#include "common.hpp"

namespace ddt {
ddtree_status check_tree(const ddtree_tree* t, const char* who);

namespace {

constexpr int kCommitThreads = 256;

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(
    ddtree_tree t, const int32_t* __restrict__ accept_len, const int32_t* __restrict__ path_nodes,
    const int32_t* __restrict__ bonus, const uint4* __restrict__ k_tree,
    const uint4* __restrict__ v_tree, int row_chunks, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache, const int64_t* __restrict__ cache_base, int64_t cache_rows,
    int capacity, int32_t* __restrict__ next_prefix_len, int32_t* __restrict__ next_root) {
  const int b = blockIdx.x, j = blockIdx.y, tid = threadIdx.x;
  const int N = t.N, D = t.D;
  const int a = accept_len[b];
  const bool valid = a >= 0 && a <= D;
  if (j == 0 && tid == 0) {
    next_prefix_len[b] = valid ? t.position[static_cast<long>(b) * N] + a + 1 : -1;
    next_root[b] = bonus[b];
  }
  if (!valid || j > a) return;
  const int node = path_nodes[static_cast<long>(b) * (D + 1) + j];
  if (node < 0 || node >= N) return;
  const int pos = t.position[static_cast<long>(b) * N + node];
  if (pos < 0 || pos >= capacity) return;
  const int64_t row = cache_base[b] + pos;
  if (row < 0 || row >= cache_rows) return;
  const long src = (static_cast<long>(b) * N + node) * row_chunks;
  const long dst = row * row_chunks;
  for (int c = tid; c < row_chunks; c += kCommitThreads) {
    const uint4 kv = k_tree[src + c];
    const uint4 vv = v_tree[src + c];
    k_cache[dst + c] = kv;
    v_cache[dst + c] = vv;
  }
}

}  // namespace
}  // namespace ddt

extern "C" ddtree_status ddtree_commit(const ddtree_tree* tree, const int32_t* accept_len,
                                       const int32_t* path_nodes, const int32_t* bonus,
                                       const void* k_tree, const void* v_tree, int32_t Hkv,
                                       int32_t Dh, ddtree_dtype dtype, void* k_cache,
                                       void* v_cache, const int64_t* cache_base,
                                       int64_t cache_rows, int32_t capacity,
                                       int32_t* next_prefix_len, int32_t* next_root,
                                       hipStream_t stream) {
  using namespace ddt;
  ddtree_status st = check_tree(tree, "ddtree_commit");
  if (st != DDTREE_OK) return st;
  if (!accept_len || !path_nodes || !bonus || !k_tree || !v_tree || !k_cache || !v_cache ||
      !cache_base || !next_prefix_len || !next_root)
    return fail(DDTREE_EINVAL, "ddtree_commit: null pointer");
  if (dtype != DDTREE_BF16 && dtype != DDTREE_F32)
    return fail(DDTREE_EINVAL, "ddtree_commit: unknown dtype %d", static_cast<int>(dtype));
  if (Hkv < 1 || Dh < 1 || cache_rows < 0 || capacity < 0)
    return fail(DDTREE_EINVAL, "ddtree_commit: Hkv=%d Dh=%d cache_rows=%lld capacity=%d", Hkv, Dh,
                static_cast<long long>(cache_rows), capacity);
  const long row_bytes = static_cast<long>(Hkv) * Dh * (dtype == DDTREE_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0)
    return fail(DDTREE_EUNSUPPORTED, "ddtree_commit: a K/V row of %ld bytes is not a multiple of 16",
                row_bytes);
  if (row_bytes / 16 > (1L << 30))
    return fail(DDTREE_EINVAL, "ddtree_commit: K/V rows of %ld bytes", row_bytes);
  if (!aligned16(k_tree) || !aligned16(v_tree) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(DDTREE_EINVAL, "ddtree_commit: tensors must be 16-byte aligned");
  const dim3 grid(tree->B, tree->D + 1);
  hipLaunchKernelGGL(commit_kernel, grid, dim3(kCommitThreads), 0, stream, *tree, accept_len,
                     path_nodes, bonus, static_cast<const uint4*>(k_tree),
                     static_cast<const uint4*>(v_tree), static_cast<int>(row_bytes / 16),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), cache_base,
                     cache_rows, capacity, next_prefix_len, next_root);
  return check_launch("ddtree_commit");
}
