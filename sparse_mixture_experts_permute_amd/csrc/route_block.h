// Device-side routing of a decode step, shared by the top-k + grouping
// kernel and the weight-streaming kernel that routes its token itself.
#pragma once
#include "common.h"

namespace moe {

// One wavefront, one token: k rounds of a wavefront arg-max over the scores
// v[j] of experts lane + 64 j (-inf past E; ties go to the lower index), then
// the gate of each pick (gate_mode: 0 softmax over the selected, 1 softmax
// over all E, 2 sigmoid of each, 3 entropy-aware: see below).  selv / seli:
// this wave's LDS rows for the picks.  Writes idx / gate [k] of the token.
//
// Entropy-aware routing ("Mixtral 8x7B model architecture", section 4.1):
// p = softmax(v / tau) over all E with tau = 0.1; the token keeps k experts
// when the entropy -sum p ln p exceeds 0.8, else k - 1 (the page's 3 and 2;
// per token, see the reading of that page), the gates are the selected p as
// they are, and an empty slot gets idx -1 (placed nowhere) and gate 0.  The
// entropy is evaluated as ln z - (sum w u) / z with u = (v - max) / tau,
// w = exp(u), z = sum w, so a probability that underflows contributes 0.
// gate_mode 4 (the page's listing: one k for the batch, the largest per-token
// k): the same, except that a slot past the token's own k keeps its
// probability and holds -(e + 2) for its expert e, so that a later pass
// over the batch (entropy_batch_kernel) can keep or empty it.
constexpr float ENTROPY_TAU = 0.1f;
constexpr float ENTROPY_THRESHOLD = 0.8f;
__device__ __forceinline__ void wave_topk_gate(const float (&v)[4], int E, int k, int gate_mode,
                                               float *selv, int *seli, int32_t *__restrict__ idx,
                                               float *__restrict__ gate) {
  const int lane = lane_id();
  unsigned taken = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + kWave * j;
      if (e < E && !(taken & (1u << j)) && (bi == 0x7fffffff || v[j] > bv)) {
        bv = v[j];
        bi = e;
      }
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == 0) {
      selv[r] = bv;
      seli[r] = bi;
    }
  }
  // lane 0's selections become visible to the whole wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const float m = selv[0];  // the largest score of the token
  float z = 0.f;
  if (gate_mode == 0) {
    // softmax over the k selected scores
    for (int r = lane; r < k; r += kWave) z += expf(selv[r] - m);
  } else if (gate_mode == 1) {
    // softmax over all E scores (v[] holds -inf past E)
#pragma unroll
    for (int j = 0; j < 4; ++j) z += expf(v[j] - m);
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) z += __shfl_xor(z, off);
  if (gate_mode == 3 || gate_mode == 4) {
    float zt = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + kWave * j < E) {
        const float u = (v[j] - m) / ENTROPY_TAU;
        const float w = expf(u);
        zt += w;
        s1 += w * u;
      }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      zt += __shfl_xor(zt, off);
      s1 += __shfl_xor(s1, off);
    }
    const float H = logf(zt) - s1 / zt;
    const int kt = H > ENTROPY_THRESHOLD ? k : k - 1;
    for (int r = lane; r < k; r += kWave) {
      const float p = expf((selv[r] - m) / ENTROPY_TAU) / zt;
      if (gate_mode == 4) {
        idx[r] = r < kt ? seli[r] : -(seli[r] + 2);
        gate[r] = p;
      } else {
        idx[r] = r < kt ? seli[r] : -1;
        gate[r] = r < kt ? p : 0.f;
      }
    }
    return;
  }
  for (int r = lane; r < k; r += kWave) {
    idx[r] = seli[r];
    const float l = selv[r];
    // gate_mode 2: logistic sigmoid of the selected score on its own
    gate[r] = gate_mode == 2 ? 1.0f / (1.0f + expf(-l)) : expf(l - m) / z;
  }
}

// Where the grouping of a decode step's pairs goes (global or LDS memory).
struct RouteOut {
  int32_t *counts, *offsets, *perm, *inv, *mtiles0, *mtiles1, *shared_seg, *active;
};

// Grouping of the P = T * k pairs of a decode step by expert, by one
// wavefront with a lane per pair (P <= 64, E <= 64): the stable counting sort
// under the capacity (the first `capacity` pairs of an expert in pair order,
// capacity <= P), as the permutation kernels do.  sidx: the pairs' experts
// (idx -1 or any id outside [0, E): placed nowhere).  Writes counts [E],
// offsets / mtiles0 / mtiles1 [E + 1], perm [kept pairs], inv [P], active
// [nactive] and active[E] = nactive, shared_seg [8].
__device__ __forceinline__ void wave_group_pairs(const int32_t *sidx, int T, int E, int k,
                                                 int capacity, int bm0, int bm1,
                                                 const RouteOut &o) {
  const int lane = lane_id();
  const int P = T * k;
  const int ev = lane < P ? sidx[lane] : -1;
  const bool valid = (unsigned)ev < (unsigned)E;  // an empty slot (idx -1) is placed nowhere
  const int e = valid ? ev : 0;
  // lanes holding the same expert: intersect ballots over the bits of e (< 64)
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 6; ++bit) {
    const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? ones : ~ones;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int rank = __popcll(same & below);  // earlier pairs of the same expert
  // lane x < E: pairs of expert x, kept pairs, m-tiles, and exclusive prefixes
  int hist = 0;
  for (int x = 0; x < E; ++x) {
    const int n = __popcll(__ballot(valid && e == x));
    if (lane == x) hist = n;
  }
  const int c = lane < E ? min(hist, capacity) : 0;
  const int c0 = (c + bm0 - 1) / bm0, c1 = (c + bm1 - 1) / bm1, ca = c > 0 ? 1 : 0;
  int s_c = c, s_0 = c0, s_1 = c1, s_a = ca;  // inclusive scans over the lanes
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int u_c = __shfl_up(s_c, off), u_0 = __shfl_up(s_0, off);
    const int u_1 = __shfl_up(s_1, off), u_a = __shfl_up(s_a, off);
    if (lane >= off) {
      s_c += u_c;
      s_0 += u_0;
      s_1 += u_1;
      s_a += u_a;
    }
  }
  if (lane < E) {
    o.counts[lane] = c;
    o.offsets[lane] = s_c - c;
    o.mtiles0[lane] = s_0 - c0;
    o.mtiles1[lane] = s_1 - c1;
    if (c > 0) o.active[s_a - 1] = lane;
  }
  if (lane == E - 1) {
    o.offsets[E] = s_c;
    o.mtiles0[E] = s_0;
    o.mtiles1[E] = s_1;
    o.active[E] = s_a;
  }
  const int first = __shfl(s_c - c, e);  // the expert's first slot
  if (valid) {
    if (rank < capacity) {
      o.perm[first + rank] = lane;
      o.inv[lane] = first + rank;
    } else {
      o.inv[lane] = -1;
    }
  } else if (lane < P) {
    o.inv[lane] = -1;
  }
  if (lane == 0) {
    o.shared_seg[0] = 0;
    o.shared_seg[1] = T;
    o.shared_seg[2] = 0;
    o.shared_seg[3] = (T + bm0 - 1) / bm0;
    o.shared_seg[4] = 0;
    o.shared_seg[5] = (T + bm1 - 1) / bm1;
    o.shared_seg[6] = 0;
    o.shared_seg[7] = 1;
  }
}

}  // namespace moe
