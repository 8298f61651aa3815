// Routing of many tokens at once for the prefill gate's epilogue (gfx950):
// 16 lanes per token, four tokens per wavefront, the six steps of the
// activation/top-k epilogue (commit e0f60b9f, dsv4/kernels/router/__init__.py)
// with the selection rule and output order of the one-token router
// (wave_route_regs).
#pragma once

#include "nvfp4_device.hpp"

namespace nvr {

// score_key of a sum s + b with s a sigmoid (+0 or more): such a sum is
// never -0 (x + (-x) and +0 + -0 round to +0), so the -0 fold is not needed.
__device__ __forceinline__ uint32_t sum_key(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return max(k, 1u);
}

// Throughput routing for many tokens: 16 lanes (one DPP row) per token, four
// tokens per wavefront at once. Same six steps, selection rule and order as
// wave_route_regs. Lane l of a row holds the J16 consecutive experts
// l J16 .. l J16 + J16 - 1, read with 16-byte LDS loads (rows of logits and
// the bias must be readable up to 16 J16 entries).
//  1. keys as in wave_route_regs; lm = the lane's largest key;
//  2. for k <= 16 the k-th largest of the 16 lane maxima is a lower bound on
//     the k-th largest key (k distinct experts reach it). Each lane counts
//     the lanes above it over 15 DPP row rotations; the bound is the smallest
//     lane maximum with fewer than k lanes above it. Everything at or above
//     it survives: usually k or a few more;
//  3. for k > 16, or when more than 32 survive (flat or tied scores), the
//     exact k-th largest key K is found bit by bit from the top (32 row
//     counts of keys >= t); the keys equal to K beyond the lowest-index ones
//     that complete k are zeroed, and the survivors are the keys >= K:
//     exactly k of them;
//  4. either way a survivor is a key above one threshold, so compaction is
//     one compare per key: the survivors (at most 32) are placed by a row
//     prefix sum of the per-lane counts and each is ranked against all of
//     them with one batch of LDS reads. Only the chosen experts recompute
//     their sigmoid (from the logits row) for the weights; the weight sum is
//     a DPP row sum and each chosen lane stores its output at its rank.
constexpr int kRow16MaxSurvivors = 32;

// Entry kRow16MaxSurvivors of each row is a spare slot that absorbs the
// writes of non-surviving keys, so compaction needs no branch per key. One
// scratch serves NSET sets of four rows. A candidate is (key << 32) | ~expert.
template <int J16, int NSET>
struct Row16Scratch {
  uint64_t cand[NSET][4][kRow16MaxSurvivors + 1];
};

__device__ __forceinline__ uint32_t row_min_u32(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  return v;
}

__device__ __forceinline__ float row_sum(float v) {
  v += __int_as_float(dpp_i<kDppXor1>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppXor2>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(v)));
  v += __int_as_float(dpp_i<kDppMirror>(__float_as_int(v)));
  return v;
}

__device__ __forceinline__ int row_sum_i(int v) {
  v += dpp_i<kDppXor1>(v);
  v += dpp_i<kDppXor2>(v);
  v += dpp_i<kDppHalfMirror>(v);
  v += dpp_i<kDppMirror>(v);
  return v;
}

// Inclusive prefix sum over the 16 lanes of each DPP row.
__device__ __forceinline__ int row_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  return v;
}

// Number of lanes of the row whose value exceeds this lane's (row_ror:R).
template <int R>
__device__ __forceinline__ int count_above(uint32_t v, int n) {
  if constexpr (R < 16) return count_above<R + 1>(v, n + (dpp_u<0x120 + R>(v) > v ? 1 : 0));
  return n;
}

// Survivors 0..NS-1 of each row (entries past the count are zero), ranked
// and stored; NS = 16 or 32, lane l16 takes survivors l16 and l16 + 16.
// The chosen experts' scores are recomputed from the logits rows (the same
// sigmoid_fast of the same value, so the same bits as the keys were built
// from).
template <int J16, int NSET, int NS>
__device__ __forceinline__ void row16_rank_store(const float* const (&Lrow)[NSET], const int (&C)[NSET], int k,
                                                 float routed_scale, const bool (&valid)[NSET], int l16, int rq,
                                                 int32_t* const (&out_idx)[NSET], float* const (&out_w)[NSET],
                                                 const Row16Scratch<J16, NSET>& sc) {
  uint64_t mine[NSET][NS / 16];
  int rank[NSET][NS / 16];
#pragma unroll
  for (int r = 0; r < NSET; ++r)
#pragma unroll
    for (int h = 0; h < NS / 16; ++h) {
      mine[r][h] = sc.cand[r][rq][l16 + 16 * h];
      rank[r][h] = 0;
    }
#pragma unroll
  for (int u = 0; u < NS; ++u)
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      const uint64_t other = sc.cand[r][rq][u];
#pragma unroll
      for (int h = 0; h < NS / 16; ++h) rank[r][h] += other > mine[r][h] ? 1 : 0;
    }
  float part[NSET], ms[NSET][NS / 16];
  bool chosen[NSET][NS / 16];
#pragma unroll
  for (int r = 0; r < NSET; ++r) {
    part[r] = 0.0f;
#pragma unroll
    for (int h = 0; h < NS / 16; ++h) {
      chosen[r][h] = l16 + 16 * h < C[r] && rank[r][h] < k;
      // Entries past the count are zero (expert ~0): read expert 0 instead.
      const uint32_t e = chosen[r][h] ? 0xFFFFFFFFu - (uint32_t)mine[r][h] : 0u;
      ms[r][h] = sigmoid_fast(Lrow[r][e]);
      part[r] += chosen[r][h] ? ms[r][h] : 0.0f;
    }
  }
#pragma unroll
  for (int r = 0; r < NSET; ++r) {
    const float f = routed_scale * __builtin_amdgcn_rcpf(row_sum(part[r]));
#pragma unroll
    for (int h = 0; h < NS / 16; ++h)
      if (valid[r] && chosen[r][h]) {
        out_idx[r][rank[r][h]] = (int)(0xFFFFFFFFu - (uint32_t)mine[r][h]);
        out_w[r][rank[r][h]] = ms[r][h] * f;
      }
  }
}

// Largest per-row survivor count over the four rows of every set.
template <int NSET>
__device__ __forceinline__ int rows_max(const int (&C)[NSET]) {
  int m = 0;
#pragma unroll
  for (int r = 0; r < NSET; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) m = max(m, (int)__builtin_amdgcn_readlane(C[r], 16 * q));
  return m;
}

// Routes NSET independent sets of four rows at once (lane l16 of row group
// rq of set r reads Lrow[r]); the sets' instruction streams interleave, which
// hides the latency of each set's dependent steps.
template <int J16, int NSET>
__device__ __forceinline__ void row16_route(const float* const (&Lrow)[NSET], const float* bias_lds, int E, int k,
                                            float routed_scale, const bool (&valid)[NSET],
                                            int32_t* const (&out_idx)[NSET], float* const (&out_w)[NSET],
                                            Row16Scratch<J16, NSET>& sc) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, rq = lane >> 4;
  const int e0 = l16 * J16;
  uint32_t key[NSET][J16];
  uint32_t lm[NSET];
#pragma unroll
  for (int r = 0; r < NSET; ++r) lm[r] = 0u;
#pragma unroll
  for (int j4 = 0; j4 < J16 / 4; ++j4) {
    const float4 B4 = *reinterpret_cast<const float4*>(bias_lds + e0 + 4 * j4);
    const float Bv[4] = {B4.x, B4.y, B4.z, B4.w};
    // The 4 NSET keys of this group of experts, one stage at a time (the
    // operations of sigmoid_fast, then the bias and the key): each stage's
    // results are pinned before the next starts, so the independent chains
    // interleave; left to itself the compiler runs each key's chain to the
    // end through one register, and with one wavefront per SIMD every
    // dependent step (two transcendentals among them) then waits. Every
    // lane computes every key, masked afterwards (inside the select the
    // sigmoid was sunk into a branch per key).
    float v[NSET][4];
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      const float4 L4 = *reinterpret_cast<const float4*>(Lrow[r] + e0 + 4 * j4);
      v[r][0] = L4.x;
      v[r][1] = L4.y;
      v[r][2] = L4.z;
      v[r][3] = L4.w;
    }
    auto pin = [&]() {
#pragma unroll
      for (int r = 0; r < NSET; ++r) asm volatile("" : "+v"(v[r][0]), "+v"(v[r][1]), "+v"(v[r][2]), "+v"(v[r][3]));
    };
    auto stage = [&](auto f) {
#pragma unroll
      for (int r = 0; r < NSET; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[r][i] = f(v[r][i], i);
      pin();
    };
    stage([](float x, int) { return __builtin_amdgcn_exp2f(-1.4426950408889634f * x); });
    stage([](float x, int) { return __builtin_amdgcn_rcpf(1.0f + x); });  // = sigmoid_fast(L)
    stage([&](float x, int i) { return x + Bv[i]; });
#pragma unroll
    for (int r = 0; r < NSET; ++r)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 4 * j4 + i;
        key[r][j] = (e0 + j < E && valid[r]) ? sum_key(v[r][i]) : 0u;
        lm[r] = max(lm[r], key[r][j]);
      }
  }
  // Survivors: the keys above hi (never key 0, as hi >= 0). The bound: hi =
  // tau - 1; the exact search: hi = K - 1, after zeroing the keys equal to K
  // that this lane may not take (ties go to the lower experts: lanes in
  // order, then each lane's experts in order).
  uint32_t hi[NSET];
  int C[NSET];
#pragma unroll
  for (int r = 0; r < NSET; ++r) {
    hi[r] = 0u;
    C[r] = kRow16MaxSurvivors + 1;
  }
  auto count = [&](int r) {
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < J16; ++j) cnt += key[r][j] > hi[r] ? 1 : 0;
    return cnt;
  };
  int cnt[NSET];
  if (k <= 16) {
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      const int above = count_above<1>(lm[r], 0);
      const uint32_t tau = row_min_u32(above < k ? lm[r] : 0xFFFFFFFFu);
      hi[r] = tau > 0u ? tau - 1u : 0u;  // key > hi <=> key >= tau, for the nonzero keys
      cnt[r] = count(r);
      C[r] = row_sum_i(cnt[r]);
    }
  }
  if (rows_max<NSET>(C) > kRow16MaxSurvivors) {
    // Exact k-th largest key K of each row, bit by bit: the largest t with at
    // least k keys >= t.
    uint32_t K[NSET];
#pragma unroll
    for (int r = 0; r < NSET; ++r) K[r] = 0u;
    for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
      for (int r = 0; r < NSET; ++r) {
        const uint32_t t = K[r] | (1u << bit);
        int c = 0;
#pragma unroll
        for (int j = 0; j < J16; ++j) c += key[r][j] >= t ? 1 : 0;
        if (row_sum_i(c) >= k) K[r] = t;
      }
    }
#pragma unroll
    for (int r = 0; r < NSET; ++r) {
      int gt = 0, eq = 0;
#pragma unroll
      for (int j = 0; j < J16; ++j) {
        gt += key[r][j] > K[r] ? 1 : 0;
        eq += (key[r][j] == K[r] && key[r][j] != 0u) ? 1 : 0;
      }
      int ties = k - row_sum_i(gt);   // equal keys still to take, lowest index first
      ties -= row_scan(eq) - eq;      // minus equal keys in lanes before this one
#pragma unroll
      for (int j = 0; j < J16; ++j) {
        const bool e = key[r][j] == K[r];
        if (e && ties <= 0) key[r][j] = 0u;
        ties -= e ? 1 : 0;
      }
      hi[r] = K[r] > 0u ? K[r] - 1u : 0u;
      cnt[r] = count(r);
      C[r] = row_sum_i(cnt[r]);
    }
  }
  // Compact the survivors (at most 32 per row): a row prefix sum gives each
  // lane its first slot; keys that do not survive write the spare slot.
#pragma unroll
  for (int r = 0; r < NSET; ++r) {
    int pos = row_scan(cnt[r]) - cnt[r];
#pragma unroll
    for (int j = 0; j < J16; ++j) {
      const bool surv = key[r][j] > hi[r];
      sc.cand[r][rq][surv ? pos : kRow16MaxSurvivors] =
          ((uint64_t)key[r][j] << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(e0 + j));
      pos += surv ? 1 : 0;
    }
  }
  const int ns = rows_max<NSET>(C) <= 16 ? 16 : 32;
  // Entries past the count rank below everything.
#pragma unroll
  for (int r = 0; r < NSET; ++r) {
    sc.cand[r][rq][C[r] <= l16 ? l16 : kRow16MaxSurvivors] = 0ull;
    if (ns == 32) sc.cand[r][rq][C[r] <= l16 + 16 ? l16 + 16 : kRow16MaxSurvivors] = 0ull;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if (ns == 16) row16_rank_store<J16, NSET, 16>(Lrow, C, k, routed_scale, valid, l16, rq, out_idx, out_w, sc);
  else row16_rank_store<J16, NSET, 32>(Lrow, C, k, routed_scale, valid, l16, rq, out_idx, out_w, sc);
}

}  // namespace nvr
