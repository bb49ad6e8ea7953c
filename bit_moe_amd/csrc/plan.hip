// Dispatch plan: per-expert counts, exclusive offsets, the pair permutation
// grouped by expert (stable), the ascending union of selected experts, and
// the list of M-tiles for the grouped GEMM.
//
// "Feature Request: support DeepSeek V4.1 Flash with bounded SSD expert
// caching", §Stack progress (request-union planning, original-id remaps) and
// "Strata-DSV4.1", §Latest (10-14) (a verify pass serves the union of its
// experts once per layer).  Everything stays on the device: no host sync.
//
// Three kernels over chunks of 64 tokens (one wave per chunk):
//  plan_count    per-chunk expert histogram (LDS atomics: counts are
//                order-independent); out-of-range ids and repeats of an
//                expert within a token are left out and recorded
//  plan_scan     one block: per-expert prefix over chunks, exclusive scan over
//                experts, union compaction, GEMM tile offsets
//  plan_scatter  per chunk, the tokens in order: each pair takes the next
//                slot of its expert (the chunk's base inside the expert's
//                group, from plan_scan), which keeps the order stable.
#include "common.h"
#include "internal.h"

namespace bm {


__global__ void __launch_bounds__(64) plan_count_kernel(const int32_t *__restrict__ ids, int T, int k, int E,
                                                        int32_t *__restrict__ chunk_counts, int64_t *status) {
  extern __shared__ int32_t hist[];  // [E]
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const int t = chunk * 64 + threadIdx.x;
  if (t < T) {
    const int32_t *row = ids + int64_t(t) * k;
    for (int j = 0; j < k; ++j) {
      const int e = row[j];
      if (e < 0 || e >= E)
        record_fault(status, FAULT_BAD_EXPERT, int64_t(t) * k + j);
      else if (repeats_earlier(row, j, e))
        record_fault(status, FAULT_DUP_EXPERT, int64_t(t) * k + j);
      else
        atomicAdd(&hist[e], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 64) chunk_counts[int64_t(chunk) * E + e] = hist[e];
}

// One block of 1024 threads.  Thread e owns expert e (E <= 1024).
__global__ void __launch_bounds__(1024) plan_scan_kernel(int n_chunks, int E, int bm_tile, int bm_tile2, PlanBufs p) {
  __shared__ int32_t s_cnt[1024];
  __shared__ int32_t s_flag[1024];
  __shared__ int32_t s_tiles[1024];
  __shared__ int32_t s_tiles2[1024];
  const int e = threadIdx.x;
  int32_t total = 0;
  if (e < E) {
    // chunks in batches of 16: all of a batch's loads are issued before its
    // stores, so their latencies overlap
    for (int c0 = 0; c0 < n_chunks; c0 += 16) {
      int32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = p.chunk_counts[int64_t(min(c0 + i, n_chunks - 1)) * E + e];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (c0 + i >= n_chunks) break;
        p.chunk_counts[int64_t(c0 + i) * E + e] = total;  // base of chunk c inside expert e's group
        total += v[i];
      }
    }
  }
  s_cnt[e] = e < E ? total : 0;
  s_flag[e] = (e < E && total > 0) ? 1 : 0;
  s_tiles[e] = (e < E && bm_tile > 0) ? (total + bm_tile - 1) / bm_tile : 0;
  s_tiles2[e] = (e < E && bm_tile2 > 0) ? (total + bm_tile2 - 1) / bm_tile2 : 0;
  __syncthreads();
  // Hillis-Steele inclusive scans over 1024 entries
  for (int o = 1; o < 1024; o <<= 1) {
    int32_t a = 0, b = 0, c = 0, d = 0;
    if (e >= o) {
      a = s_cnt[e - o];
      b = s_flag[e - o];
      c = s_tiles[e - o];
      d = s_tiles2[e - o];
    }
    __syncthreads();
    s_cnt[e] += a;
    s_flag[e] += b;
    s_tiles[e] += c;
    s_tiles2[e] += d;
    __syncthreads();
  }
  if (e < E) {
    p.counts[e] = total;
    p.offsets[e + 1] = s_cnt[e];
    if (e == 0) p.offsets[0] = 0;
    if (total > 0) p.union_ids[s_flag[e] - 1] = e;
    if (p.tile_off) {
      p.tile_off[e + 1] = s_tiles[e];
      if (e == 0) p.tile_off[0] = 0;
    }
    if (p.tile_off2) {
      p.tile_off2[e + 1] = s_tiles2[e];
      if (e == 0) p.tile_off2[0] = 0;
    }
    if (e == E - 1) *p.n_union = s_flag[e];
  }
}

__global__ void __launch_bounds__(64) plan_scatter_kernel(const int32_t *__restrict__ ids, int T, int k, int E,
                                                          PlanBufs p) {
  extern __shared__ int32_t s_pos[];  // [E] next slot of each expert, then [64 * k] the chunk's ids
  int32_t *s_ids = s_pos + E;
  const int chunk = blockIdx.x;
  const int t0 = chunk * 64;
  const int nt = min(64, T - t0);
  // every load of a batch is issued before its stores, so their latencies overlap
  for (int e0 = 0; e0 < E; e0 += 64 * 8) {
    int32_t o[8], c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = min(e0 + 64 * i + int(threadIdx.x), E - 1);
      o[i] = p.offsets[e];
      c[i] = p.chunk_counts[int64_t(chunk) * E + e];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + 64 * i + threadIdx.x;
      if (e < E) s_pos[e] = o[i] + c[i];
    }
  }
  for (int i0 = 0; i0 < nt * k; i0 += 64 * 8) {
    int32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ids[int64_t(t0) * k + min(i0 + 64 * i + int(threadIdx.x), nt * k - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ii = i0 + 64 * i + threadIdx.x;
      if (ii < nt * k) s_ids[ii] = v[i];
    }
  }
  __syncthreads();
  // which pairs are served (in range, first slot of their expert in the
  // token), one token per thread; a pair that is not gets id -1
  if (int(threadIdx.x) < nt) {
    int32_t *row = s_ids + threadIdx.x * k;
    int32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = j < k ? row[j] : -1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      bool keep = v[j] >= 0 && v[j] < E;
#pragma unroll
      for (int i = 0; i < j; ++i) keep = keep && v[i] != v[j];
      if (!keep) row[j] = -1;
    }
  }
  __syncthreads();
  // tokens of the chunk in order, lane j taking slot j: the k lanes of a step
  // advance distinct counters and each expert's pairs land in token order
  // (stable).  The lane's ids are read ahead in groups of 16 tokens.
  const int j = threadIdx.x;
  if (j >= k) return;
  for (int u0 = 0; u0 < nt; u0 += 16) {
    int32_t ev[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ev[i] = s_ids[min(u0 + i, nt - 1) * k + j];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int u = u0 + i, e = ev[i];
      if (u >= nt) break;
      if (e < 0) continue;
      const int pos = s_pos[e];
      s_pos[e] = pos + 1;
      p.perm[pos] = (t0 + u) * k + j;
    }
  }
}

hipError_t launch_plan(const int32_t *ids, int T, int k, int E, int bm_tile, int bm_tile2, PlanBufs p,
                       hipStream_t stream) {
  const int n_chunks = (T + 63) / 64;
  BM_LAUNCH("plan_count_kernel", plan_count_kernel, dim3(n_chunks), dim3(64), E * sizeof(int32_t), stream, ids, T, k, E,
                     p.chunk_counts, p.status);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  BM_LAUNCH("plan_scan_kernel", plan_scan_kernel, dim3(1), dim3(1024), 0, stream, n_chunks, E, bm_tile, bm_tile2, p);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  BM_LAUNCH("plan_scatter_kernel", plan_scatter_kernel, dim3(n_chunks), dim3(64), (E + 64 * k) * sizeof(int32_t), stream,
            ids, T, k, E, p);
  return hipGetLastError();
}

size_t plan_scratch_bytes(int T, int E) {
  const size_t n_chunks = size_t(T + 63) / 64;
  return n_chunks * size_t(E) * sizeof(int32_t);
}

}  // namespace bm
