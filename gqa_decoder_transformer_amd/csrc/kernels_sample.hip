// Sampling after the LM head ("ember internals", section "sampler"): temperature,
// top-k, top-p against a temporary softmax, the final softmax with its uniform fallback,
// and an inverse-CDF draw with its argmax fallback, in that order. One block of 1024
// threads per row; every pass re-reads the row of logits (coalesced, from L2).
//
// Both masks are thresholds on z = logit / t (IEEE division, as the f32 definition), so
// after them a token survives iff z >= thr:
// * top-k (0 < k < V): thr is the k-th largest z, found exactly by an MSB-first radix
//   select over order-preserving 32-bit keys (digits of 11, 11 and 10 bits, counts in
//   LDS, the digit chosen by a block scan of the bin counts). Ties with it survive.
// * top-p (0 < p < 1): the temporary probabilities exp(z - m) / S are monotone in z, so
//   the nucleus cutoff -- the largest probability v with sum(prob >= v) > p -- is the
//   largest key z* whose survivors' weight sum exceeds p * S. The same radix search finds
//   it with weights exp(z - m) in 2^-40 fixed point (integer sums: the decision does not
//   depend on the order of the additions). When no key qualifies nothing is masked.
// Neither mask removes the maximum m, so the final softmax keeps m. The draw compares
// u * S2 with the running sum of exp(z - m) over survivors in index order (S2 = their
// total): per-256-element tile sums, a scan of the tile sums, then one wave scans the
// tile that holds the crossing. A row whose every z is -inf is drawn uniformly; when
// rounding leaves no crossing the last index holding the maximum is returned.
// Temperature 0 is the greedy argmax and never reaches this kernel.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kST = 1024;                   // threads per row
constexpr int kSW = kST / kWave;            // waves per block
constexpr int kUnroll = 8;                  // loads in flight per thread
constexpr int kTile = 4 * kWave;            // elements per tile: 4 groups of 64 lanes
constexpr int kBins = 2048;                 // 11-bit digits

static_assert(kSampleMaxVocab <= kSampleMaxTiles * kTile, "tile table too small");

typedef unsigned long long u64;

struct Smem {
  u64 hist[kBins];
  float tile_sum[kSampleMaxTiles];          // weight of each tile
  float tile_pre[kSampleMaxTiles];          // running sum before each tile
  u64 wtot[kSW];
  float redf[kSW];
  int redi[kSW];
  u64 sel[3];                               // chosen bin, new 'above', found
  float total;
  int hit;
};

EMBER_DEV float from_ordered_key(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

EMBER_DEV float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kSW; ++i) r = fmaxf(r, red[i]);
  return r;
}

EMBER_DEV int block_min_i(int v, int* red, bool want_max = false) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int n = __shfl_xor(v, o);
    v = want_max ? max(v, n) : min(v, n);
  }
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
  for (int i = 1; i < kSW; ++i) r = want_max ? max(r, red[i]) : min(r, red[i]);
  return r;
}

EMBER_DEV u64 block_sum_u64(u64 v, u64* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  u64 r = 0;
  for (int i = 0; i < kSW; ++i) r += red[i];
  return r;
}

// Inclusive scan over the block in thread order.
EMBER_DEV u64 block_scan_u64(u64 v, u64* red) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const u64 n = __shfl_up(v, o);
    if (l >= o) v += n;
  }
  __syncthreads();
  if (l == kWave - 1) red[w] = v;
  __syncthreads();
  u64 add = 0;
  for (int i = 0; i < w; ++i) add += red[i];
  return v + add;
}

EMBER_DEV float wave_scan_f32(float v) {
  const int l = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const float n = __shfl_up(v, o);
    if (l >= o) v += n;
  }
  return v;
}

// Calls f(i, value) for every i < V owned by this thread (i = threadIdx.x + j * kST),
// kUnroll loads issued before any use.
template <typename F>
EMBER_DEV void for_row(const float* L, int V, F&& f) {
  int i = threadIdx.x;
  for (; i + (kUnroll - 1) * kST < V; i += kUnroll * kST) {
    float v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = L[i + u * kST];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) f(i + u * kST, v[u]);
  }
  for (; i < V; i += kST) f(i, L[i]);
}

EMBER_DEV void zero_hist(Smem& s) {
  for (int b = threadIdx.x; b < kBins; b += kST) s.hist[b] = 0;
}

// The first bin from the top whose inclusive suffix weight, on top of `above`, exceeds T
// (nb bins of the current digit). Returns false when the total does not exceed T.
EMBER_DEV bool pick_bin(Smem& s, int nb, u64 above, u64 T, uint32_t& bin, u64& new_above) {
  __syncthreads();                                   // histogram complete
  const int hi = nb - 1 - 2 * (int)threadIdx.x, lo = hi - 1;
  const u64 whi = hi >= 0 ? s.hist[hi] : 0, wlo = lo >= 0 ? s.hist[lo] : 0;
  const u64 incl = block_scan_u64(whi + wlo, s.wtot);
  const u64 before = above + incl - whi - wlo;        // weight of the bins above hi
  if (hi >= 0 && before <= T && before + whi > T) {
    s.sel[0] = (u64)hi; s.sel[1] = before; s.sel[2] = 1;
  } else if (lo >= 0 && before + whi <= T && before + whi + wlo > T) {
    s.sel[0] = (u64)lo; s.sel[1] = before + whi; s.sel[2] = 1;
  }
  __syncthreads();
  const bool found = s.sel[2] != 0;
  bin = (uint32_t)s.sel[0];
  new_above = s.sel[1];
  __syncthreads();
  if (threadIdx.x == 0) s.sel[2] = 0;                // read by the next pick after a sync
  return found;
}

// Radix search over the keys of z for the largest key with weight(keys >= it) > T. The
// level-0 histogram is already in s.hist; `weight(z)` gives the later levels' weights.
template <typename Wt>
EMBER_DEV bool radix_search(Smem& s, const float* L, int V, float t, u64 T, Wt&& weight,
                            uint32_t& key_out) {
  uint32_t bin;
  u64 above = 0, na;
  if (!pick_bin(s, kBins, 0, T, bin, na)) return false;
  uint32_t prefix = bin << 21, pmask = 0x7FFu << 21;
  above = na;
  for (int level = 1; level < 3; ++level) {
    const int shift = level == 1 ? 10 : 0;
    const uint32_t dmask = level == 1 ? 0x7FFu : 0x3FFu;
    zero_hist(s);
    __syncthreads();
    for_row(L, V, [&](int i, float l) {
      const float z = l / t;
      const uint32_t key = ordered_key(z);
      if ((key & pmask) == prefix) {
        const u64 w = weight(z);
        if (w) atomicAdd(&s.hist[(key >> shift) & dmask], w);
      }
    });
    // the chosen bin's weight carries over, so a bin is always found at this level
    if (!pick_bin(s, (int)dmask + 1, above, T, bin, na)) break;
    prefix |= bin << shift;
    pmask |= dmask << shift;
    above = na;
  }
  key_out = prefix;
  return true;
}

__global__ void __launch_bounds__(kST) k_sample(SampleArgs a) {
  __shared__ Smem s;
  const int r = blockIdx.x;
  const int V = a.V;
  const float t = a.temperature;
  const float* L = a.logits + (size_t)r * a.ld;
  const bool topk = a.top_k > 0 && a.top_k < V;
  const bool topp = a.top_p > 0.f && a.top_p < 1.f;
  if (threadIdx.x < 3) s.sel[threadIdx.x] = 0;
  zero_hist(s);
  __syncthreads();

  // ---- pass 1: max of z (NaN flagged and skipped), level-0 counts for top-k
  float m = -INFINITY;
  bool nan = false;
  for_row(L, V, [&](int i, float l) {
    const float z = l / t;
    nan |= z != z;
    m = fmaxf(m, z);
    if (topk && z == z) atomicAdd(&s.hist[ordered_key(z) >> 21], 1ull);
  });
  if (nan && a.flags) a.flags[kFlagNaN] = 1;
  m = block_max(m, s.redf);
  const bool uniform = m == -INFINITY;               // every z is -inf (or NaN)

  // ---- top-k: thr = the k-th largest z
  float thr = -INFINITY;
  if (topk) {
    uint32_t key;
    if (radix_search(s, L, V, t, (u64)(a.top_k - 1),
                     [](float z) -> u64 { return z == z ? 1ull : 0ull; }, key))
      thr = from_ordered_key(key);
  }

  // ---- top-p: thr = the largest z whose survivors' weight exceeds p * S
  if (topp && !uniform) {
    zero_hist(s);
    __syncthreads();
    const float scale = 1099511627776.0f;            // 2^40
    auto weight = [&](float z) -> u64 {
      return z >= thr ? (u64)(expf(z - m) * scale) : 0ull;
    };
    u64 tot = 0;
    for_row(L, V, [&](int i, float l) {
      const float z = l / t;
      const u64 w = weight(z);
      if (w) {
        atomicAdd(&s.hist[ordered_key(z) >> 21], w);
        tot += w;
      }
    });
    tot = block_sum_u64(tot, s.wtot);
    const u64 T = (u64)((double)a.top_p * (double)tot);
    uint32_t key;
    if (radix_search(s, L, V, t, T, weight, key)) thr = fmaxf(thr, from_ordered_key(key));
  }

  // ---- final distribution: e(i) = exp(z - m) for z >= thr (1 for a uniform row)
  auto e_of = [&](float l) -> float {
    if (uniform) return 1.f;
    const float z = l / t;
    return z >= thr ? expf(z - m) : 0.f;
  };
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int ntiles = (V + kTile - 1) / kTile;
  for (int t0 = wv; t0 < ntiles; t0 += 4 * kSW) {   // 4 tiles (16 loads) in flight
    float v[4][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        v[q][g] = L[min((t0 + q * kSW) * kTile + g * kWave + lane, V - 1)];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int tile = t0 + q * kSW;
      if (tile >= ntiles) break;
      float acc = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g)
        acc += tile * kTile + g * kWave + lane < V ? e_of(v[q][g]) : 0.f;
      acc = wave_sum_uniform(acc);
      if (lane == 0) s.tile_sum[tile] = acc;
    }
  }
  __syncthreads();
  if (wv == 0) {                                     // running sums before each tile
    float carry = 0.f;
    for (int g0 = 0; g0 < ntiles; g0 += kWave) {
      const int j = g0 + lane;
      const float x = j < ntiles ? s.tile_sum[j] : 0.f;
      const float inc = wave_scan_f32(x);
      const float up = __shfl_up(inc, 1);          // every lane takes part in the shuffle
      const float exc = lane == 0 ? 0.f : up;
      if (j < ntiles) s.tile_pre[j] = carry + exc;
      carry += __shfl(inc, kWave - 1);
    }
    if (lane == 0) s.total = carry;
  }
  __syncthreads();
  const float S2 = s.total;
  const int did = a.d_pos ? *a.d_pos : a.pos;
  const int urow = min(max(did, 0), a.u_rows - 1);
  const float u = a.uniform[(size_t)urow * a.u_ld + a.col0 + r];
  const float target = u * S2;
  // the first weighted tile whose running sum at its end exceeds the target
  int first = ntiles;
  for (int tile = threadIdx.x; tile < ntiles; tile += kST) {
    const float end = tile + 1 < ntiles ? s.tile_pre[tile + 1] : S2;
    if (s.tile_sum[tile] > 0.f && end > target && first == ntiles) first = tile;
  }
  first = block_min_i(first, s.redi);
  int hit = -1;
  if (first < ntiles) {
    if (wv == 0) {
      const float pre = s.tile_pre[first];
      const int base = first * kTile + lane;
      float run = 0.f;
      int found = -1, last_nz = -1;
      for (int g = 0; g < 4; ++g) {
        const int i = base + g * kWave;
        const float e = i < V ? e_of(L[min(i, V - 1)]) : 0.f;
        const float inc = wave_scan_f32(e);
        const unsigned long long cross = __ballot(e > 0.f && pre + (run + inc) > target);
        const unsigned long long nz = __ballot(e > 0.f);
        if (found < 0 && cross) found = g * kWave + __ffsll((long long)cross) - 1;
        if (nz) last_nz = g * kWave + 63 - __clzll((long long)nz);
        run += __shfl(inc, kWave - 1);
      }
      // rounding between the tile sum and the scan: the tile's last weighted element
      if (lane == 0) s.hit = first * kTile + (found >= 0 ? found : last_nz);
    }
    __syncthreads();
    hit = s.hit;
  }
  if (hit < 0) {                                     // no crossing: the last maximum
    int last = -1;
    for_row(L, V, [&](int i, float l) {
      const float z = l / t;
      if (uniform || (z == m && z >= thr)) last = i;
    });
    hit = block_min_i(last, s.redi, true);
  }
  if (threadIdx.x == 0) a.next[r] = min(max(hit, 0), V - 1);
}

}  // namespace

void launch_sample(const SampleArgs& a, hipStream_t st) {
  if (a.R <= 0 || a.V <= 0) return;
  hipLaunchKernelGGL(k_sample, dim3(a.R), dim3(kST), 0, st, a);
}

}  // namespace ember
