// Decode-path job bookkeeping shared by the GEMV and MFMA decode kernels:
// a routed job is one expert of the ascending union of the call's valid
// expert ids together with the (token, slot) pairs routed to it; the shared
// job covers every token.
#pragma once

#include "common.h"
#include "internal.h"

namespace bm {

struct Job {
  int e;           // expert (-1: shared)
  int n;           // tokens (pairs) of the job, <= 8 (decode takes T <= 8)
  uint64_t pairs;  // pair indices t*k + j, 8 bits each (shared job: token indices)
};

// i-th pair / token of a job (shifts instead of array indexing keep the job in
// registers)
BM_DEVICE int jpair(const Job &job, int i) { return int((job.pairs >> (8 * i)) & 0xFFu); }
BM_DEVICE int jtok(const FfnArgs &a, const Job &job, int i) {
  return job.e < 0 ? jpair(job, i) : jpair(job, i) / a.k;
}

// Routed job of pair slot p: expert e = ids[p] with every pair served by it,
// or false when pair p is not served (id out of range, or a repeat of an
// expert earlier in its token's slots) or an earlier served pair already
// chose e (so each expert of the union is one job and its weights are read
// once).  Served pairs of one expert belong to distinct tokens, so a job has
// at most T <= 8 of them.  All loads are uniform across the block (scalar).
BM_DEVICE bool pair_served(const FfnArgs &a, int q) {
  const int e = a.ids[q];
  return e >= 0 && e < a.E && !repeats_earlier(a.ids + (q / a.k) * a.k, q % a.k, e);
}

BM_DEVICE bool pair_job(const FfnArgs &a, int p, Job &job) {
  const int P = a.T * a.k;
  if (!pair_served(a, p)) return false;
  const int e = a.ids[p];
  job.e = e;
  job.n = 0;
  job.pairs = 0;
  for (int q = 0; q < P; ++q) {
    if (a.ids[q] != e || !pair_served(a, q)) continue;
    if (q < p) return false;  // not the first served occurrence
    if (job.n < 8) job.pairs |= uint64_t(q) << (8 * job.n);
    ++job.n;
  }
  if (job.n > 8) job.n = 8;  // unreachable: one served pair per token and T <= 8
  return true;
}

// pair_job computed by each wave on its own: the call's pair ids are read by
// the lanes (T * k <= 64) together with the block's own id, each lane finds
// whether its pair repeats an earlier slot of its token (k - 1 lane
// shuffles), and the served pairs of e are matched with one ballot, so the job
// costs one round trip to memory.
BM_DEVICE bool pair_job_wave(const FfnArgs &a, int p, Job &job) {
  const int P = a.T * a.k;
  if (P > 64) return pair_job(a, p, job);
  const int lane = threadIdx.x & 63;
  int id = lane < P ? a.ids[lane] : -1;
  if (id < 0 || id >= a.E) id = -1;
  const int slot = lane % a.k;
  bool dup = false;
  for (int d = 1; d < a.k; ++d) {
    const int prev = __shfl(id, (lane - d) & 63);
    dup = dup || (slot >= d && prev == id);
  }
  if (dup) id = -1;  // not served
  const int e = __builtin_amdgcn_readlane(id, p);  // ids[p] when pair p is served
  if (e < 0) return false;
  uint64_t m = __ballot(id == e);
  if (m & ((uint64_t(1) << p) - 1)) return false;  // an earlier served pair chose e
  job.e = e;
  job.n = 0;
  job.pairs = 0;
  while (m != 0 && job.n < 8) {
    const int q = __builtin_ctzll(m);
    m &= m - 1;
    job.pairs |= uint64_t(q) << (8 * job.n);
    ++job.n;
  }
  return true;
}

BM_DEVICE void shared_job(const FfnArgs &a, Job &job) {
  job.e = -1;
  job.n = a.T;
  job.pairs = 0x0706050403020100ull;
}

}  // namespace bm
