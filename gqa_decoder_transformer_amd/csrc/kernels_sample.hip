// Sampling after the LM head ("ember internals", section "sampler"): temperature,
// top-k, top-p against a temporary softmax, the final softmax with its uniform fallback,
// and an inverse-CDF draw with its argmax fallback, in that order.
//
// Both masks are thresholds on z = logit / t (IEEE division, as the f32 definition), so
// after them a token survives iff z >= thr:
// * top-k (0 < k < V): thr is the k-th largest z, found exactly by an MSB-first radix
//   select over order-preserving 32-bit keys (digits of 11, 11 and 10 bits). Ties with
//   it survive.
// * top-p (0 < p < 1): the temporary probabilities exp(z - m) / S are monotone in z, so
//   the nucleus cutoff -- the largest probability v with sum(prob >= v) > p -- is the
//   largest key z* whose survivors' weight sum exceeds p * S. The same radix search finds
//   it with weights exp(z - m) in 2^-40 fixed point (integer sums: the decision does not
//   depend on the order of the additions). When no key qualifies nothing is masked.
// Neither mask removes the maximum m, so the final softmax keeps m. The draw compares
// u * S2 with the running sum of exp(z - m) over survivors in index order (S2 = their
// total): 256-token tile sums, a scan of the tile sums, then one wave scans the tile that
// holds the crossing. A row whose every z is -inf is drawn uniformly; when rounding
// leaves no crossing the last index holding the maximum is returned.
//
// Layout of the work: each row is cut into chunks of 2048 tokens, one 256-thread block
// per chunk (a row of a 152k vocabulary spreads over ~75 CUs). A draw is a sequence of
// phase launches -- max and top-k digit 0, top-k digits 1 and 2, top-p digits 0..2, tile
// sums and the draw -- of which only the enabled stages run. Within a phase every block
// adds its LDS histogram to the row's global one with device-scope atomics; the last
// block to finish (a per-row counter) takes the phase's decision, clears what it
// consumed and leaves the result in the row's state for the next launch. No block ever
// waits for another.
// Temperature 0 is the greedy argmax and never reaches these kernels.
#include "common.h"
#include "kernels.h"

namespace ember {

namespace {

constexpr int kSB = 256;                    // threads per block
constexpr int kSWv = kSB / kWave;           // waves per block
constexpr int kPer = kSampleChunk / kSB;    // tokens per thread (one per 256-token tile)
constexpr int kBins = kSampleBins;

static_assert(kPer == 8 && kSB == 256, "one token per thread and 256-token tile");
static_assert(kBins % kSB == 0 && kSampleMaxTiles % kSB == 0, "work per thread");

typedef unsigned long long u64;

enum Phase { PH_MAX_K0 = 0, PH_K1 = 1, PH_K2 = 2, PH_P0 = 3, PH_P1 = 4, PH_P2 = 5, PH_DRAW = 6 };

EMBER_DEV float from_ordered_key(uint32_t k) {
  const uint32_t b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(b);
}

// A load served by L2, where the other blocks' atomics and fenced stores are visible.
template <typename T>
EMBER_DEV T load_l2(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan of v over the block in thread order (red: kSWv entries).
template <typename T>
EMBER_DEV T block_scan(T v, T* red) {
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const T n = __shfl_up(v, o);
    if (l >= o) v += n;
  }
  __syncthreads();
  if (l == kWave - 1) red[w] = v;
  __syncthreads();
  T add = 0;
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

template <typename T, typename Op>
EMBER_DEV T block_reduce(T v, T* red, Op op) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  T r = red[0];
  for (int i = 1; i < kSWv; ++i) r = op(r, red[i]);
  return r;
}

// The on-device draw of batch row `row` for the token predicted from position `pos`
// (when the caller passes no draws): the first output word of Philox4x32-10 (Salmon,
// Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
// (pos, row, 0, 0) and key (seed mod 2^32, seed div 2^32), as (word >> 8) * 2^-24.
// Philox4x32-10 rounds: the products M0 c0 and M1 c2 (high and low words) give the next
// counter (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key moves
// by the Weyl constants between rounds. Only the first output word is kept.
EMBER_DEV float sample_philox_u(unsigned long long seed, uint32_t pos, uint32_t row) {
  uint32_t c0 = pos, c1 = row, c2 = 0u, c3 = 0u;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    if (rnd) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const unsigned long long p0 = (unsigned long long)0xD2511F53u * c0;
    const unsigned long long p1 = (unsigned long long)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  return (float)(c0 >> 8) * 0x1p-24f;
}


struct Shared {
  union {
    u64 hist[kBins];                                  // digit histogram of the block
    struct {
      float sum[kSampleMaxTiles];
      float pre[kSampleMaxTiles];
    } tile;
  } u;
  u64 redu[kSWv];
  float redf[kSWv * kPer];
  int redi[kSWv];
  u64 pick_above;
  float thread_off[kSB];
  float total;
  uint32_t pick_bin;
  int pick_found;
  int last;
  int hit;
};

// Count this block done; true in the block that finishes the phase last, which also
// re-arms the counter for the next phase. Every value a block hands to the last one
// travels through a device-scope atomic (histogram adds, the maximum, tile sums stored
// with device scope) and is read back with device-scope loads, so no cache writeback or
// invalidation is needed: waiting for the block's memory operations to complete before
// the counter's add orders them (a device-scope fence here costs ~4 us per launch).
EMBER_DEV bool finish_phase(SampleState& st, Shared& s) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);                      // vm, exp and lgkm counts all zero
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&st.count, 1u);
    s.last = old == gridDim.x - 1;
    if (s.last) atomicExch(&st.count, 0u);
  }
  __syncthreads();
  return s.last;
}

// Adds the block's LDS histogram to a global one.
template <typename G>
EMBER_DEV void merge_hist(Shared& s, G* g, int nb) {
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kSB) {
    const u64 v = s.u.hist[b];
    if (v) atomicAdd(&g[b], (G)v);
  }
}

// Last block: the first bin from the top of the global histogram g (nb bins of the digit
// at `shift`) whose inclusive suffix weight, on top of the weight above the prefix,
// exceeds T. Extends the row's prefix with it; `live` = whether one was found. Clears g.
template <typename G>
EMBER_DEV void pick_digit(Shared& s, SampleState& st, G* g, int nb, int shift, u64 T, bool level0,
                          int& live) {
  const int bpt = nb / kSB;                           // 8 or 4 bins per thread, descending
  u64 w[kBins / kSB];
  u64 sum = 0;
  for (int q = 0; q < bpt; ++q) {
    const int b = nb - 1 - ((int)threadIdx.x * bpt + q);
    w[q] = (u64)load_l2(&g[b]);
    sum += w[q];
  }
  if (threadIdx.x == 0) s.pick_found = 0;
  const u64 above = level0 ? 0ull : st.above;
  const u64 incl = block_scan(sum, s.redu);           // its syncs order pick_found
  u64 run = above + incl - sum;
  for (int q = 0; q < bpt; ++q) {
    if (run <= T && run + w[q] > T) {
      s.pick_bin = (uint32_t)(nb - 1 - ((int)threadIdx.x * bpt + q));
      s.pick_above = run;
      s.pick_found = 1;
    }
    run += w[q];
  }
  for (int q = 0; q < bpt; ++q) g[nb - 1 - ((int)threadIdx.x * bpt + q)] = 0;
  __syncthreads();
  live = s.pick_found;
  if (threadIdx.x == 0 && live) {
    const uint32_t dmask = (uint32_t)nb - 1u;
    st.prefix = (level0 ? 0u : st.prefix) | (s.pick_bin << shift);
    st.pmask = (level0 ? 0u : st.pmask) | (dmask << shift);
    st.above = s.pick_above;
  }
}

template <int PH>
__global__ void __launch_bounds__(kSB) k_sample_phase(SampleArgs a) {
  __shared__ Shared s;
  const int r = blockIdx.y;
  const int V = a.V;
  SampleState& st = a.state[r];
  const float* L = a.logits + (size_t)r * a.ld;
  const float t = a.temperature;
  const int base = blockIdx.x * kSampleChunk + threadIdx.x;
  const bool topk = a.top_k > 0 && a.top_k < V;

  // this thread's tokens: base + j * 256, i.e. token threadIdx.x of the block's tile j
  float z[kPer];
  bool in[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = base + j * kSB;
    in[j] = i < V;
    z[j] = L[min(i, V - 1)] / t;
  }

  if constexpr (PH == PH_MAX_K0) {
    if (topk) {
      for (int b = threadIdx.x; b < kBins; b += kSB) s.u.hist[b] = 0;
      __syncthreads();
    }
    float m = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (!in[j]) continue;
      nan |= z[j] != z[j];
      m = fmaxf(m, z[j]);
      if (topk && z[j] == z[j]) atomicAdd(&s.u.hist[ordered_key(z[j]) >> 21], 1ull);
    }
    if (nan && a.flags) a.flags[kFlagNaN] = 1;
    m = block_reduce(m, s.redf, [](float x, float y) { return fmaxf(x, y); });
    if (threadIdx.x == 0) atomicMax(&st.maxkey, ordered_key(m));
    if (topk) merge_hist(s, st.hist_k[0], kBins);
    if (!finish_phase(st, s)) return;
    int live = 0;
    if (topk) pick_digit(s, st, st.hist_k[0], kBins, 21, (u64)(a.top_k - 1), true, live);
    if (threadIdx.x == 0) {
      st.thr = -INFINITY;
      st.live_k = live;
      st.live_p = 0;
    }
  } else if constexpr (PH == PH_DRAW) {
    const float m = from_ordered_key(load_l2(&st.maxkey));
    const bool uniform = m == -INFINITY;
    const float thr = st.thr;
    auto weight = [&](float zz) -> float {
      if (uniform) return 1.f;
      return zz >= thr ? expf(zz - m) : 0.f;
    };
    // tile sums: tile j of this block holds token threadIdx.x of every thread
    const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const float ws = wave_sum_uniform(in[j] ? weight(z[j]) : 0.f);
      if (lane == 0) s.redf[wv * kPer + j] = ws;
    }
    __syncthreads();
    const int tld = sample_tiles_ld(V);
    if (threadIdx.x < kPer) {
      const int j = threadIdx.x;
      float sum = 0.f;
      for (int w = 0; w < kSWv; ++w) sum += s.redf[w * kPer + j];
      __hip_atomic_store(&a.tiles[(size_t)r * tld + blockIdx.x * kPer + j], sum, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!finish_phase(st, s)) return;

    // ---- the last block of the row: running sums before each tile, then the draw.
    // Sequential within each thread's 16 tiles and along the threads' totals, so the
    // sums never decrease and the end of the last weighted tile is exactly the total.
    const int ntiles = gridDim.x * kPer;
    const float* tiles = a.tiles + (size_t)r * tld;
    constexpr int kTPT = kSampleMaxTiles / kSB;       // tiles per thread
    const int nthr = (ntiles + kTPT - 1) / kTPT;
    float local = 0.f;
    for (int q = 0; q < kTPT; ++q) {
      const int j = threadIdx.x * kTPT + q;
      if (j < ntiles) {
        const float v = load_l2(&tiles[j]);
        s.u.tile.sum[j] = v;
        s.u.tile.pre[j] = local;                      // this thread's part, offset later
        local += v;
      }
    }
    s.thread_off[threadIdx.x] = local;
    __syncthreads();
    if (threadIdx.x == 0) {
      float off = 0.f;
      for (int i = 0; i < nthr; ++i) {
        const float v = s.thread_off[i];
        s.thread_off[i] = off;
        off += v;
      }
      s.total = off;
    }
    __syncthreads();
    {
      const float off = s.thread_off[threadIdx.x];
      for (int q = 0; q < kTPT; ++q) {
        const int j = threadIdx.x * kTPT + q;
        if (j < ntiles) s.u.tile.pre[j] = off + s.u.tile.pre[j];
      }
    }
    __syncthreads();
    const float S2 = s.total;
    const int did = a.d_pos ? a.d_pos[r] : a.pos;
    float u;
    if (a.uniform) {
      const int urow = min(max(did, 0), a.u_rows - 1);
      u = a.uniform[(size_t)urow * a.u_ld + a.col0 + r];
    } else {
      u = sample_philox_u(a.seed, (uint32_t)max(did, 0), (uint32_t)(a.col0 + r));
    }
    const float target = u * S2;
    // the first weighted tile whose running sum at its end exceeds the target
    int first = ntiles;
    for (int j = threadIdx.x; j < ntiles; j += kSB) {
      const float end = j + 1 < ntiles ? s.u.tile.pre[j + 1] : S2;
      if (s.u.tile.sum[j] > 0.f && end > target && first == ntiles) first = j;
    }
    first = block_reduce(first, s.redi, [](int x, int y) { return x < y ? x : y; });
    int hit = -1;
    if (first < ntiles) {
      if (wv == 0) {
        const float pre = s.u.tile.pre[first];
        float acc = 0.f;
        int found = -1, last_nz = -1;
        for (int g = 0; g < kSB / kWave; ++g) {
          const int i = first * kSB + g * kWave + lane;
          const float e = i < V ? weight(L[min(i, V - 1)] / t) : 0.f;
          const float inc = wave_scan_f32(e);
          const unsigned long long cross = __ballot(e > 0.f && pre + (acc + inc) > target);
          const unsigned long long nz = __ballot(e > 0.f);
          if (found < 0 && cross) found = g * kWave + __ffsll((long long)cross) - 1;
          if (nz) last_nz = g * kWave + 63 - __clzll((long long)nz);
          acc += __shfl(inc, kWave - 1);
        }
        // rounding between the tile sum and the scan: the tile's last weighted token
        if (lane == 0) s.hit = first * kSB + (found >= 0 ? found : last_nz);
      }
      __syncthreads();
      hit = s.hit;
    }
    if (hit < 0) {                                    // no crossing: the last maximum
      int lastm = -1;
      for (int i = threadIdx.x; i < V; i += kSB) {
        const float zz = L[i] / t;
        if (uniform || (zz == m && zz >= thr)) lastm = i;
      }
      hit = block_reduce(lastm, s.redi, [](int x, int y) { return x > y ? x : y; });
    }
    if (threadIdx.x == 0) {
      a.next[r] = min(max(hit, 0), V - 1);
      st.maxkey = 0;                                  // clean state for the next draw
      st.ptotal = 0;
    }
  } else {                                            // a later radix digit of either mask
    constexpr bool is_p = PH >= PH_P0;
    constexpr int level = is_p ? PH - PH_P0 : PH - PH_MAX_K0;
    constexpr int shift = level == 0 ? 21 : (level == 1 ? 10 : 0);
    constexpr int nb = level == 2 ? 1024 : kBins;
    const float m = from_ordered_key(load_l2(&st.maxkey));
    if (is_p && m == -INFINITY) return;               // every z is -inf: drawn uniformly
    if (level > 0 && !(is_p ? st.live_p : st.live_k)) return;
    const uint32_t prefix = level > 0 ? st.prefix : 0u, pmask = level > 0 ? st.pmask : 0u;
    const float thr = st.thr;
    for (int b = threadIdx.x; b < nb; b += kSB) s.u.hist[b] = 0;
    __syncthreads();
    u64 tot = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (!in[j] || z[j] != z[j]) continue;
      const uint32_t key = ordered_key(z[j]);
      if ((key & pmask) != prefix) continue;
      u64 w = 1;
      if (is_p) {
        w = z[j] >= thr ? (u64)(expf(z[j] - m) * 1099511627776.0f) : 0ull;   // 2^40
        tot += w;
      }
      if (w) atomicAdd(&s.u.hist[(key >> shift) & (uint32_t)(nb - 1)], w);
    }
    if (is_p && level == 0) {
      tot = block_reduce(tot, s.redu, [](u64 x, u64 y) { return x + y; });
      if (threadIdx.x == 0 && tot) atomicAdd(&st.ptotal, tot);
    }
    if constexpr (is_p)
      merge_hist(s, st.hist_p[level], nb);
    else
      merge_hist(s, st.hist_k[level], nb);
    if (!finish_phase(st, s)) return;
    // p * S in the same fixed point (S: every survivor's weight)
    const u64 T = is_p ? (u64)((double)a.top_p * (double)load_l2(&st.ptotal))
                       : (u64)(a.top_k - 1);
    int live = 0;
    if constexpr (is_p)
      pick_digit(s, st, st.hist_p[level], nb, shift, T, level == 0, live);
    else
      pick_digit(s, st, st.hist_k[level], nb, shift, T, level == 0, live);
    __syncthreads();
    if (threadIdx.x == 0) {
      if (is_p) st.live_p = live; else st.live_k = live;
      // after the last digit the prefix is the key itself; a search that ran dry on a
      // later digit (not expected: the chosen bin's weight carries over) keeps the
      // prefix so far, a lower bound
      if ((level == 2 && live) || (!live && level > 0)) {
        const float key = from_ordered_key(st.prefix);
        st.thr = is_p ? fmaxf(st.thr, key) : key;
      }
    }
  }
}

}  // namespace

void launch_sample(const SampleArgs& a, hipStream_t st) {
  if (a.R <= 0 || a.V <= 0) return;
  const dim3 grid(sample_blocks(a.V), a.R);
  const bool topk = a.top_k > 0 && a.top_k < a.V;
  const bool topp = a.top_p > 0.f && a.top_p < 1.f;
  hipLaunchKernelGGL(k_sample_phase<PH_MAX_K0>, grid, dim3(kSB), 0, st, a);
  if (topk) {
    hipLaunchKernelGGL(k_sample_phase<PH_K1>, grid, dim3(kSB), 0, st, a);
    hipLaunchKernelGGL(k_sample_phase<PH_K2>, grid, dim3(kSB), 0, st, a);
  }
  if (topp) {
    hipLaunchKernelGGL(k_sample_phase<PH_P0>, grid, dim3(kSB), 0, st, a);
    hipLaunchKernelGGL(k_sample_phase<PH_P1>, grid, dim3(kSB), 0, st, a);
    hipLaunchKernelGGL(k_sample_phase<PH_P2>, grid, dim3(kSB), 0, st, a);
  }
  hipLaunchKernelGGL(k_sample_phase<PH_DRAW>, grid, dim3(kSB), 0, st, a);
}

}  // namespace ember
