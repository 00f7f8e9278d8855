// Top-k selection of one token's router logits by one wavefront, shared by the top-k
// kernel of the router and the decode-sized layer kernels.
//
// Pages: MarkTechPost, "Perplexity open sources Lily, a Rust + Metal inference engine for
// Qwen3.6-35B-A3B on Apple Silicon", body paragraph 4 (a router scores 256 experts and
// picks eight).  The weighting (softmax over the selected logits) and the tie rule (equal
// logits go to the lower expert id) are readings; the pages state neither.
//
// The wavefront ranks the fp32 logits by a 64-bit key (order-preserving float bits, then
// the complemented expert id so equal logits rank the lower id higher) and extracts the
// k+1 best.  If the k-th and (k+1)-th fp32 logits are closer than `tau`, the experts at
// least tau above L_(k+1) keep their places, and every expert within tau of L_(k+1) is
// rescored exactly in fp64 (bf16 x fp32 products are exact in fp64); the best of those,
// by fp64 logit, fill the remaining places.  As long as the fp32 error is under tau/2 the
// experts above are in the exact top k and those below are not, so the selection equals
// the exact (fp64) top-k.  Runs of selected experts whose neighbours are closer than tau
// are then rescored in fp64 and sorted, so the order is the exact descending order too.
#pragma once

#include "common.h"

namespace moeq4 {
__device__ __forceinline__ uint32_t ordered_bits(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unordered_bits(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
__device__ __forceinline__ uint64_t ordered_bits64(double v) {
  uint64_t u = (uint64_t)__double_as_longlong(v);
  return (u & 0x8000000000000000ull) ? ~u : (u | 0x8000000000000000ull);
}

// Wavefront reductions with DPP, the result on every lane: within each row of 16 lanes
// (quad swaps, then rotations by 4 and 8), then the row results carried to lane 63 by
// the row broadcasts of lane 15 and lane 31, read back as a scalar.  Lanes a DPP step
// does not update contribute the identity.  The order of the additions is fixed.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp(uint32_t v, uint32_t identity, Op op) {
  const int id = (int)identity;
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(id, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_dpp(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ __forceinline__ float wave_max_f32(float v) {
  return __uint_as_float(wave_reduce_dpp(__float_as_uint(v), 0xFF800000u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  return __uint_as_float(wave_reduce_dpp(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}

// Butterfly reductions with the result in every lane, no scalar round trip: within each
// row of 16 lanes (quad swaps, then rotations by 4 and 8), then across row pairs and
// halves with the gfx950 lane swaps (each returns the two values a lane and its partner
// hold; op takes both).
template <typename Op>
__device__ __forceinline__ uint32_t wave_all_reduce(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));  // row_ror:4
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));  // row_ror:8
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // rows r, r ^ 1
  v = op((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // halves
  return op((uint32_t)b[0], (uint32_t)b[1]);
}

// Sum over the wavefront in fp64 with the same bits on every lane: partners of lane i are
// i ^ 1 and i ^ 2 (quad permutes), then the other quad of its half-row and the other half
// of its row (half-row and row mirrors, which pair whole quads and halves once the values
// are uniform within them), then the neighbouring row and half (lane swaps).  Each step
// adds two values that every lane of the pair holds, in either order, so all lanes agree.
__device__ __forceinline__ double dpp_partner_f64(double v, int ctrl_tag) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
  switch (ctrl_tag) {
    case 0:
      lo = __builtin_amdgcn_update_dpp(0, lo, 0xb1, 0xf, 0xf, false);  // quad [1,0,3,2]
      hi = __builtin_amdgcn_update_dpp(0, hi, 0xb1, 0xf, 0xf, false);
      break;
    case 1:
      lo = __builtin_amdgcn_update_dpp(0, lo, 0x4e, 0xf, 0xf, false);  // quad [2,3,0,1]
      hi = __builtin_amdgcn_update_dpp(0, hi, 0x4e, 0xf, 0xf, false);
      break;
    case 2:
      lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xf, 0xf, false);  // row_half_mirror
      hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xf, 0xf, false);
      break;
    default:
      lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xf, 0xf, false);  // row_mirror
      hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xf, 0xf, false);
      break;
  }
  return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_partner_f64(v, 0);
  v += dpp_partner_f64(v, 1);
  v += dpp_partner_f64(v, 2);
  v += dpp_partner_f64(v, 3);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const auto l16 = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
  const auto h16 = __builtin_amdgcn_permlane16_swap((uint32_t)(u >> 32), (uint32_t)(u >> 32), false, false);
  const double a = __longlong_as_double((long long)(((uint64_t)h16[0] << 32) | l16[0]));
  const double b = __longlong_as_double((long long)(((uint64_t)h16[1] << 32) | l16[1]));
  v = a + b;
  const uint64_t w = (uint64_t)__double_as_longlong(v);
  const auto l32 = __builtin_amdgcn_permlane32_swap((uint32_t)w, (uint32_t)w, false, false);
  const auto h32 = __builtin_amdgcn_permlane32_swap((uint32_t)(w >> 32), (uint32_t)(w >> 32), false, false);
  const double c = __longlong_as_double((long long)(((uint64_t)h32[0] << 32) | l32[0]));
  const double d = __longlong_as_double((long long)(((uint64_t)h32[1] << 32) | l32[1]));
  return c + d;
}

// (value, expert) pair order: larger value first, then lower expert id.
struct Cand {
  double v;
  int e;
};
__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  return a.v > b.v || (a.v == b.v && a.e < b.e);
}

// One wavefront selects the top k of one token (logits Lt [E], E <= 64 MAXC, x row xt [D],
// router R [E, D] for the fp64 rescoring).  On lane j < k: out_e = the j-th expert
// (descending logit), out_w = its routing weight (softmax over the k selected fp32
// logits); other lanes get out_w = 0.  No barriers: callable by any wavefront alone.
// Rescoring passes (E <= 256) take NB experts at a time (2 or 4) with RS 1 KB steps of x
// and their R rows in flight; RS = 8 covers d_model 2048 in one round of loads.
template <int MAXC, int RS = 4, int NB = 4>
__device__ __forceinline__ void topk_token(const float* __restrict__ Lt,
                                           const uint16_t* __restrict__ xt,
                                           const float* __restrict__ R, int D, int E, int k,
                                           float tau, int& out_e, float& out_w) {
  const int lane = threadIdx.x & 63;
  float val[MAXC];
  uint32_t key[MAXC];  // order-preserving bits of the logit (at least 1); 0 once selected
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    int e = c * 64 + lane;
    val[c] = e < E ? Lt[e] : 0.f;
    key[c] = e < E ? max(ordered_bits(val[c]), 1u) : 0u;
  }

  // Each lane first sorts its own MAXC (key, slot) pairs, best first (larger key, then the
  // lower slot, i.e. the lower expert id), with a fixed merge network.  Lane j keeps the
  // j-th selection.  A round takes the largest head of the wavefront, then the lowest
  // expert id among the lanes that hold it (two all-lane reductions); the winning lane
  // drops its head.  No branch depends on lane data.
  uint32_t sk[MAXC];
  int sc[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    sk[c] = key[c];
    sc[c] = c;
  }
  // Batcher's odd-even merge sort (MAXC a power of two): compare-exchange (i, i + d)
#pragma unroll
  for (int pw = 1; pw < MAXC; pw <<= 1)
#pragma unroll
    for (int d = pw; d >= 1; d >>= 1)
#pragma unroll
      for (int j0 = d % pw; j0 + d < MAXC; j0 += 2 * d)
#pragma unroll
        for (int i = 0; i < d; ++i) {
          const int x = i + j0, y = i + j0 + d;
          if (y < MAXC && x / (2 * pw) == y / (2 * pw)) {
            const bool swap = sk[y] > sk[x] || (sk[y] == sk[x] && sc[y] < sc[x]);
            const uint32_t kx = sk[x], ky = sk[y];
            const int cx = sc[x], cy = sc[y];
            sk[x] = swap ? ky : kx;
            sk[y] = swap ? kx : ky;
            sc[x] = swap ? cy : cx;
            sc[y] = swap ? cx : cy;
          }
        }
  int my_e = -1;
  float my_v = 0.f;
  const int nsel = (k + 1 < E) ? k + 1 : E;
  auto umax = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  auto umin = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  for (int j = 0; j < nsel; ++j) {
    const uint32_t hk = sk[0];
    const uint32_t hi = wave_all_reduce(hk, umax);
    const int e = (int)wave_all_reduce(hk == hi ? (uint32_t)(64 * sc[0] + lane) : 0xFFFFFFFFu, umin);
    const float v = unordered_bits(hi);
    my_e = lane == j ? e : my_e;
    my_v = lane == j ? v : my_v;
    const bool pop = (e & 63) == lane;
#pragma unroll
    for (int c = 0; c + 1 < MAXC; ++c) {
      sk[c] = pop ? sk[c + 1] : sk[c];
      sc[c] = pop ? sc[c + 1] : sc[c];
    }
    sk[MAXC - 1] = pop ? 0u : sk[MAXC - 1];
  }

  // fp64 logits of up to NB experts (uniform ids ce[0 .. nb-1]; slots past nb repeat
  // ce[0]) (E > 256: always four): lane d sums d, d + 64, ... in order (several steps of
  // loads in flight), then a fixed butterfly adds the lanes, so every lane gets the sums.
  // bf16 x fp32 products are exact in fp64.
  constexpr int NBE = MAXC >= 16 ? 4 : NB;
  auto exact4 = [&](const int* ce, int nb, double* out) __attribute__((always_inline)) {
    const float* Rr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) Rr[j] = R + (int64_t)(j < nb ? ce[j] : ce[0]) * D;
    double sj[4] = {0.0, 0.0, 0.0, 0.0};
    if constexpr (MAXC >= 16) {
      // lane l takes d = 64 s + l of step s, two steps in flight (registers permitting)
      constexpr int UN = 2;
      for (int d0 = 0; d0 < D; d0 += 64 * UN) {
        float xv[UN], rv[UN][4];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int d = min(d0 + 64 * u + lane, D - 1);
          xv[u] = d0 + 64 * u + lane < D ? bf16lo_to_f32(xt[d]) : 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) rv[u][j] = Rr[j][d];
        }
#pragma unroll
        for (int u = 0; u < UN; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) sj[j] += (double)xv[u] * (double)rv[u][j];
      }
    } else {
      // lane l takes d = 256 s + 4 l .. 4 l + 3 of step s (D % 64 == 0: a step's four d
      // are all in range or all out), 16-byte loads of each row, RS steps in flight
      constexpr int UN = RS;
      for (int d0 = 0; d0 < D; d0 += 256 * UN) {
        u32x2_t xv[UN];
        f32x4_t rv[UN][NBE];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int dd = d0 + 256 * u + 4 * lane;
          const int d = dd < D ? dd : D - 4;
          xv[u] = *(const u32x2_t*)(xt + d);
#pragma unroll
          for (int j = 0; j < NBE; ++j) rv[u][j] = *(const f32x4_t*)(Rr[j] + d);
          if (dd >= D) xv[u] = u32x2_t{0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const float xf[4] = {bf16lo_to_f32(xv[u][0]), bf16hi_to_f32(xv[u][0]),
                               bf16lo_to_f32(xv[u][1]), bf16hi_to_f32(xv[u][1])};
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int j = 0; j < NBE; ++j) sj[j] += (double)xf[c] * (double)rv[u][j][c];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < NBE; ++j) out[j] = wave_sum_f64_dpp(sj[j]);
  };

  if (k < E) {
    const float vk = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_v), k - 1));
    const float vk1 = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(my_v), k));
    if (vk - vk1 < tau) {
      // With an fp32 error below tau / 2: an expert whose fp32 logit is at least
      // L_(k+1) + tau is in the exact top k (it is among the fp32 top k, and only those
      // could beat it), one below L_(k+1) - tau is not (the k + 1 fp32 best beat it).
      // The first kind keep their places (a prefix of the ranking); the experts in
      // between are rescored exactly in fp64 and fill the remaining places.  Four
      // candidates per pass over x: lane d sums d, d + 64, ... in order (several steps
      // of loads in flight), then a fixed butterfly adds the lanes.
      const float thr_lo = vk1 - tau, thr_hi = vk1 + tau;
      const int n_sure = __popcll(__ballot(lane < k && my_v >= thr_hi));
      double exact[MAXC];
      bool cand[MAXC];
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        const int e = c * 64 + lane;
        cand[c] = e < E && val[c] >= thr_lo && !(val[c] >= thr_hi);
        exact[c] = 0.0;
      }
      int ce[4] = {0, 0, 0, 0}, nb = 0;  // expert ids of the pending batch (uniform)
      auto flush = [&]() __attribute__((always_inline)) {
        double sums[4];
        exact4(ce, nb, sums);
#pragma unroll
        for (int j = 0; j < NBE; ++j) {
          const double sum = sums[j];
          // selects over every slot (a branch per slot lets the compiler index the
          // array by ce[j] >> 6, which moves it to scratch memory)
          const bool hit = j < nb && (ce[j] & 63) == lane;
#pragma unroll
          for (int c = 0; c < MAXC; ++c) exact[c] = (hit && c == (ce[j] >> 6)) ? sum : exact[c];
        }
        nb = 0;
      };
#pragma unroll
      for (int c = 0; c < MAXC; ++c) {
        uint64_t mask = __ballot(cand[c]);
        while (mask) {
          const int b = __builtin_ctzll(mask);
          mask &= mask - 1;
          // ce[nb] = c * 64 + b, without a dynamically indexed array
#pragma unroll
          for (int j = 0; j < 4; ++j) ce[j] = j == nb ? c * 64 + b : ce[j];
          if (++nb == NBE) flush();
        }
      }
      if (nb > 0) flush();
      // the remaining places from the candidates by (fp64 logit desc, expert id asc)
      for (int j = n_sure; j < k; ++j) {
        Cand best{-__builtin_inf(), 0x7FFFFFFF};
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          Cand cc{exact[c], c * 64 + lane};
          if (cand[c] && better(cc, best)) best = cc;
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) {
          Cand o;
          o.v = xor_f64(best.v, msk);
          o.e = (int)xor_u32((uint32_t)best.e, msk);
          if (better(o, best)) best = o;
        }
        if (best.e >= E) best.e = 0;  // only with NaN logits (fewer than k candidates)
        // its fp32 logit from the lane that holds it (best is the same on every lane)
        float bv = 0.f;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) bv = c == (best.e >> 6) ? val[c] : bv;
        bv = __shfl(bv, best.e & 63);
        if (lane == j) {
          my_e = best.e;
          my_v = bv;
        }
        const bool won = (best.e & 63) == lane;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) cand[c] = (won && c == (best.e >> 6)) ? false : cand[c];
      }
    }
  }

  // The selected set is exact; so is its order wherever adjacent fp32 logits are at least
  // tau apart.  Runs of selected experts whose neighbours are closer than that are
  // rescored in fp64 and sorted within the run by (fp64 logit desc, expert id asc), with
  // an odd-even transposition sort over the lanes of the run, so the order equals the
  // exact descending order whenever the fp32 error is below tau / 2.
  if (k > 1) {
    const float vprev = __shfl(my_v, lane > 0 ? lane - 1 : 0);
    const float vnext = __shfl(my_v, lane + 1 < 64 ? lane + 1 : 63);
    const bool joins_prev = lane > 0 && lane < k && vprev - my_v < tau;
    const bool joins_next = lane + 1 < k && my_v - vnext < tau;
    uint64_t runs = __ballot(joins_prev || joins_next);
    if (runs) {
      const uint64_t breaks = ~__ballot(joins_prev);  // bit j: lane j starts a run
      double ex = 0.0;
      int ce[4] = {0, 0, 0, 0}, cl[4] = {0, 0, 0, 0}, nb = 0;
      while (runs) {
        const int b = __builtin_ctzll(runs);
        runs &= runs - 1;
        const int e = __builtin_amdgcn_readlane(my_e, b);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ce[j] = j == nb ? e : ce[j];
          cl[j] = j == nb ? b : cl[j];
        }
        if (++nb == NBE || runs == 0) {
          double sums[4];
          exact4(ce, nb, sums);
#pragma unroll
          for (int j = 0; j < NBE; ++j)
            if (j < nb && cl[j] == lane) ex = sums[j];
          nb = 0;
        }
      }
      for (int r = 0; r < k; ++r) {
        const int partner = ((lane & 1) == (r & 1)) ? lane + 1 : lane - 1;
        const int pl = partner < 0 ? 0 : (partner > 63 ? 63 : partner);
        const double pv = __shfl(ex, pl);
        const int pe = __shfl(my_e, pl);
        const float pf = __shfl(my_v, pl);
        const int hi = lane > partner ? lane : partner;
        const bool same = partner >= 0 && partner < k && lane < k && !((breaks >> hi) & 1ull);
        if (same) {
          const Cand a{ex, my_e}, o{pv, pe};
          // the lower lane keeps the better of the pair
          const bool take = lane < partner ? better(o, a) : better(a, o);
          if (take) {
            ex = pv;
            my_e = pe;
            my_v = pf;
          }
        }
      }
    }
  }

  // softmax over the k selected fp32 logits
  const bool mine = lane < k;
  const float mx = wave_max_f32(mine ? my_v : -__builtin_inff());
  const float z = mine ? __expf(my_v - mx) : 0.f;
  const float sum = wave_sum_f32(z);
  out_e = my_e;
  out_w = mine ? z / sum : 0.f;
}

}  // namespace moeq4
