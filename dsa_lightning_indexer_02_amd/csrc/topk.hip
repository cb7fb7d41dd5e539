// Per-query top-k selection (AMD MI355X DeepSeek-V3.2-Exp article, section "Fine-Grained Token
// Selection"; DeepSeek-V3.2-Exp summary page, section "Method": top-k = 2048): for query row t,
// the k highest scores among its n_t visible keys; equal scores go to the lower key index.
//
// When every row fits 32768 scores, each row is one workgroup of 256 threads and about 17 KB of
// LDS (six per CU), and the row is streamed from memory instead of held in registers (a second
// read of a row just read comes from the caches):
//   1. one pass over an eighth of the row samples two scores per 16-byte unit (2048 samples);
//      one histogram pass in equal-width value bins over the samples puts a pivot a safe margin
//      below the expected position of the k-th largest score;
//   2. one pass over the whole row counts the scores at or above the pivot and appends their
//      positions to an LDS candidate list (each thread walks the set bits of its compare mask);
//   3. an exact select over the candidates' scores (re-read): a histogram pass in equal-width
//      value bins (a second one inside a crowded bin) narrows the k-th largest to at most 64
//      candidates, which one wave ranks; that gives the threshold key tau and the number of its
//      copies to take (heavy ties fall back to a radix select over the keys); every element
//      >= tau is a candidate, so this is exact;
//   4. ordered emission: candidates set their position's bit in one of two LDS bitmaps (above
//      tau / equal to tau), a block scan of the bit counts gives every selected position its
//      output slot, and the index list is staged in LDS and stored with 16-byte stores.
// When the candidates cannot hold the selection (fewer than k, or more than 4096: an unlucky
// sample, heavy ties, or k itself large), the radix select and the bitmaps run over the whole
// row by streaming passes instead.  The output is deterministic: every key above the threshold
// in index order, then the lowest-index ties.
//
// Longer rows are cut into chunks of 32768, one workgroup of 512 threads per chunk with the
// chunk in registers (64 scores per thread: every chunk but a row's last is full, and the
// register form reads it once); the same sampled pivot, candidate select and bitmap emission
// give the chunk's own top-k candidates (key, index), and a merge pass (one 512-thread
// workgroup per row, candidates in registers) runs the select over the concatenated
// candidates.  This is exact: an element in the row's top-k is in its chunk's top-k under the
// same order.
#include "dsa_internal.hpp"

namespace dsa {

constexpr int TK_THREADS = 512;
constexpr int TK_WAVES = TK_THREADS / WAVE;
constexpr int TK_BINS = 2048;
constexpr int TK_DIGIT = 11;
constexpr int TK_CHUNK_EPT = 64;  // 512 * 64 = 32768 scores per workgroup
constexpr int64_t TK_CHUNK = (int64_t)TK_THREADS * TK_CHUNK_EPT;
constexpr int TK_MERGE_EPT = 16;  // 8192 candidates per merge
constexpr int TK_STAGE = 2048;    // index lists up to this length are staged in LDS

// merge kernel state
struct TopkShared {
  uint32_t hist[TK_BINS];
  int32_t stage[TK_STAGE];
  uint32_t wsum[TK_WAVES][2];
  uint32_t red[TK_WAVES][2];
  uint32_t sel_bin, sel_above, sel_cnt;
  uint32_t small[WAVE];             // keys of a bin small enough to rank in one wave
  uint32_t small_n;
  uint32_t kmax, kmin;
};

// Inverse of score_key on the keys of non-NaN scores (key 0x7FFFFFFF, never produced, reads -0.0).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Bin of score v among LIN_BINS bins of equal width 1 / scale from lo (clamped to the first and
// the last bin): monotonic in v, so a higher bin holds only larger scores and a bin's rank window
// is exact whatever the rounding of the arithmetic.
constexpr int LIN_BINS = 1024;
__device__ __forceinline__ int lin_bin(float v, float lo, float scale) {
  // clamped as a float, so the conversion is defined for every input: a scale that overflowed
  // (a range of a few ulps) gives 0 * inf = NaN -> bin 0 for v = lo and inf -> the last bin above
  return (int)fminf(fmaxf((v - lo) * scale, 0.0f), (float)(LIN_BINS - 1));
}

// Whether value bins over [lo, hi] are usable: their width must be a finite float.
__device__ __forceinline__ bool lin_range_ok(float lo, float hi) { return hi - lo < __builtin_inff(); }

// Position of element e of this thread inside the workgroup's range.
template <int EPT>
__device__ __forceinline__ int elem_pos(int wave, int lane, int e) {
  return wave * (WAVE * EPT) + (e >> 2) * (4 * WAVE) + 4 * lane + (e & 3);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
// inclusive prefix sum over the wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = (uint32_t)__shfl_up((int)v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Zero the histogram (once per workgroup; every select pass leaves it zeroed again).  The
// barrier that makes it visible is the one in block_minmax.
__device__ __forceinline__ void hist_clear(TopkShared& sh) {
  for (int i = threadIdx.x; i < TK_BINS; i += TK_THREADS) sh.hist[i] = 0;
  if (threadIdx.x == 0) sh.small_n = 0;
}

// Maximum and minimum of the valid keys (0 = no element) of the workgroup.
template <int EPT>
__device__ void block_minmax(const uint32_t (&key)[EPT], TopkShared& sh, uint32_t& mx, uint32_t& mn) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // no per-element validity test: 0 (no element) never raises the maximum, and key - 1 wraps it
  // to the top for the minimum
  mx = 0;
  mn = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    mx = max(mx, key[e]);
    mn = min(mn, key[e] - 1u);
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn) + 1u;  // 0 when the wave has no element
  if (lane == 0) {
    sh.red[wave][0] = mx;
    sh.red[wave][1] = mn;
  }
  __syncthreads();
  mx = 0;
  mn = 0xFFFFFFFFu;
  for (int i = 0; i < TK_WAVES; ++i) {
    mx = max(mx, sh.red[i][0]);
    mn = min(mn, sh.red[i][1] - 1u);
  }
  mn += 1u;
}

// One histogram pass of the radix select over the keys whose bits above shift + bits equal
// prefix, binned by the `bits`-wide digit at `shift`.  The histogram is zero on entry and again
// on exit (each thread clears the four bins it reads).  want(total) gives the rank, counted from
// the top, sought among the `total` matching keys (0: none).  Returns the digit of the bin
// holding that rank and the number of matching keys in higher bins.
template <int EPT, typename Want>
__device__ void hist_pass(const uint32_t (&key)[EPT], int shift, int bits, uint32_t prefix, TopkShared& sh,
                          Want want, uint32_t& bin, uint32_t& above_out, uint32_t* count_out = nullptr) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi_shift = shift + bits;
  const uint32_t dmask = (1u << bits) - 1u;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t kk = key[e];
    const bool match = kk != 0 && (hi_shift >= 32 ? true : ((kk >> hi_shift) == prefix));
    if (match) atomicAdd(&sh.hist[(kk >> shift) & dmask], 1u);
  }
  __syncthreads();
  // suffix counts: thread t owns the 4 bins 4*(511 - t) .. +3 (highest bins first)
  const int b0 = 4 * (TK_THREADS - 1 - tid);
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = sh.hist[b0 + i];
    sh.hist[b0 + i] = 0;
  }
  const uint32_t own = h[0] + h[1] + h[2] + h[3];
  const uint32_t incl = wave_incl_scan(own, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();
  uint32_t above = incl - own, total = 0;
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t w = sh.wsum[i][0];
    if (i < wave) above += w;
    total += w;
  }
  const uint32_t need = want(total);
  if (above < need && need <= above + own) {
    uint32_t a = above;
    for (int i = 3; i >= 0; --i) {
      if (need <= a + h[i]) {
        sh.sel_bin = (uint32_t)(b0 + i);
        sh.sel_above = a;
        sh.sel_cnt = h[i];
        break;
      }
      a += h[i];
    }
  }
  __syncthreads();
  bin = sh.sel_bin;
  above_out = sh.sel_above;
  if (count_out) *count_out = sh.sel_cnt;
}

// The end of an exact select once the bin holding the sought rank has cnt <= 64 keys: they (the
// valid keys whose bits from shift up equal prefix) are collected in LDS and one wave ranks them:
// tau is the key with fewer than `need` keys above it and at least `need` at or above it, k_rem
// the count of its copies to take.  sh.small_n is zero on entry and on exit.
template <int EPT, typename Match>
__device__ void small_finish_if(const uint32_t (&key)[EPT], Match match, uint32_t cnt, uint32_t need, TopkShared& sh,
                                uint32_t& tau, uint32_t& k_rem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t kk = key[e];
    if (kk != 0 && match(kk)) sh.small[atomicAdd(&sh.small_n, 1u)] = kk;
  }
  __syncthreads();
  if (wave == 0) {
    const uint32_t x = (uint32_t)lane < cnt ? sh.small[lane] : 0u;
    uint32_t gt = 0, eq = 0;
    const uint32_t cu = (uint32_t)__builtin_amdgcn_readfirstlane((int)cnt);  // workgroup-uniform
    for (uint32_t m = 0; m < cu; ++m) {
      const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)m);  // lane m holds small[m]
      gt += y > x;
      eq += y == x;
    }
    if ((uint32_t)lane < cnt && gt < need && need <= gt + eq) {  // every copy of tau writes the same
      sh.sel_bin = x;
      sh.sel_above = need - gt;
    }
    if (lane == 0) sh.small_n = 0;
  }
  __syncthreads();
  tau = sh.sel_bin;
  k_rem = sh.sel_above;
}

template <int EPT>
__device__ void small_finish(const uint32_t (&key)[EPT], int shift, uint32_t prefix, uint32_t cnt, uint32_t need,
                             TopkShared& sh, uint32_t& tau, uint32_t& k_rem) {
  small_finish_if<EPT>(key, [&](uint32_t kk) { return (kk >> shift) == prefix; }, cnt, need, sh, tau, k_rem);
}

// Exact threshold search given the maximum mx and a lower bound mn (>= 1) of the valid keys
// (keys 0 are no element; the valid ones all share the bits above the highest bit where mx and
// mn differ).  Returns tau (the k-th largest key) and k_rem (how many elements equal to tau are
// selected).  Requires at least k valid elements and a zero histogram.
template <int EPT>
__device__ void radix_select(const uint32_t (&key)[EPT], uint32_t k, uint32_t mx, uint32_t mn, TopkShared& sh,
                             uint32_t& tau, uint32_t& k_rem) {
  if (mx == mn) {  // every valid element is equal
    tau = mx;
    k_rem = k;
    return;
  }
  const int hb = 31 - __clz(mx ^ mn);
  int shift = hb >= TK_DIGIT - 1 ? hb - (TK_DIGIT - 1) : 0;
  int bits = hb - shift + 1;
  uint32_t prefix = (hb == 31) ? 0u : (mx >> (hb + 1));  // bits above the window
  uint32_t need = k;
  while (true) {
    uint32_t bin, above, cnt;
    hist_pass<EPT>(key, shift, bits, prefix, sh, [&](uint32_t) { return need; }, bin, above, &cnt);
    need -= above;
    prefix = (shift + bits >= 32 ? 0u : (prefix << bits)) | bin;
    if (shift == 0) break;
    if (cnt <= (uint32_t)WAVE) {  // workgroup-uniform
      small_finish<EPT>(key, shift, prefix, cnt, need, sh, tau, k_rem);
      return;
    }
    bits = shift >= TK_DIGIT ? TK_DIGIT : shift;
    shift -= bits;
  }
  tau = prefix;
  k_rem = need;
}

// One histogram pass over the scores of the valid keys that match(), in LIN_BINS bins of width
// 1 / scale from lo (lo and scale finite): the bin holding the need-th largest of them (1 <= need
// <= their count), the matching keys above it and in it.  The histogram is zero on entry and on
// exit.
constexpr int TK_LPT = LIN_BINS / TK_THREADS;  // bins per thread in the suffix scan
template <int EPT, typename Match>
__device__ void lin_pass(const uint32_t (&key)[EPT], Match match, float lo, float scale, uint32_t need,
                         TopkShared& sh, int& bin, uint32_t& above_out, uint32_t& cnt_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t kk = key[e];
    if (kk != 0 && match(kk)) atomicAdd(&sh.hist[lin_bin(key_score(kk), lo, scale)], 1u);
  }
  __syncthreads();
  const int b0 = TK_LPT * (TK_THREADS - 1 - tid);  // the highest bins first
  uint32_t h[TK_LPT];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < TK_LPT; ++i) {
    h[i] = sh.hist[b0 + i];
    sh.hist[b0 + i] = 0;
    own += h[i];
  }
  const uint32_t incl = wave_incl_scan(own, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();
  uint32_t above = incl - own;
  for (int i = 0; i < wave; ++i) above += sh.wsum[i][0];
  if (above < need && need <= above + own) {
    uint32_t a = above;
    for (int i = TK_LPT - 1; i >= 0; --i) {
      if (need <= a + h[i]) {
        sh.sel_bin = (uint32_t)(b0 + i);
        sh.sel_above = a;
        sh.sel_cnt = h[i];
        break;
      }
      a += h[i];
    }
  }
  __syncthreads();
  bin = (int)sh.sel_bin;
  above_out = sh.sel_above;
  cnt_out = sh.sel_cnt;
}

// Exact select as radix_select, starting with LIN_BINS equal-width bins over the value range
// [key_score(mn), key_score(mx)] and one refinement of the bin holding the k-th largest; once that
// bin has at most 64 keys one wave ranks them.  Heavier ties fall back to the radix select.
template <int EPT>
__device__ void lin_select(const uint32_t (&key)[EPT], uint32_t k, uint32_t mx, uint32_t mn, TopkShared& sh,
                           uint32_t& tau, uint32_t& k_rem) {
  const float lo = key_score(mn), hi = key_score(mx);
  if (mx != mn && lin_range_ok(lo, hi)) {  // workgroup-uniform
    const float scale = (float)LIN_BINS / (hi - lo);
    int b;
    uint32_t above, cnt;
    lin_pass<EPT>(key, [](uint32_t) { return true; }, lo, scale, k, sh, b, above, cnt);
    auto in_b = [&](uint32_t kk) { return lin_bin(key_score(kk), lo, scale) == b; };
    if (cnt <= (uint32_t)WAVE) {
      small_finish_if<EPT>(key, in_b, cnt, k - above, sh, tau, k_rem);
      return;
    }
    const float lo2 = lo + (float)b / scale, scale2 = scale * (float)LIN_BINS;
    int b2;
    uint32_t above2, cnt2;
    lin_pass<EPT>(key, in_b, lo2, scale2, k - above, sh, b2, above2, cnt2);
    if (cnt2 <= (uint32_t)WAVE) {
      small_finish_if<EPT>(
          key, [&](uint32_t kk) { return in_b(kk) && lin_bin(key_score(kk), lo2, scale2) == b2; }, cnt2,
          k - above - above2, sh, tau, k_rem);
      return;
    }
  }
  radix_select<EPT>(key, k, mx, mn, sh, tau, k_rem);
}

// Number of set bits of a wave mask held by lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m, uint32_t acc) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, acc));
}

// Ordered emission of the selected elements: all keys > tau in position order, then the
// first k_rem keys == tau.  emit(pos, slot) is called once per selected element.  The selection
// is first reduced to two bit masks per thread (bit e: element e), so the emission loop does not
// index the key array.  Within a group of 4 WAVE positions (4 lane + c), the rank of an element
// is the number of selected elements of lower lanes (ballots, mbcnt) plus this lane's selected
// elements of lower c.
template <int EPT, typename Emit>
__device__ void emit_selected(const uint32_t (&key)[EPT], uint32_t tau, uint32_t k, uint32_t k_rem,
                              TopkShared& sh, Emit emit) {
  static_assert(EPT <= 64 && EPT % 4 == 0, "one 64-bit mask per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t gtm = 0, eqm = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    gtm |= (uint64_t)(key[e] > tau) << e;
    eqm |= (uint64_t)(key[e] == tau) << e;
  }
  // wave totals
  uint32_t tg = (uint32_t)__builtin_popcountll(gtm), te = (uint32_t)__builtin_popcountll(eqm);
  for (int o = 32; o > 0; o >>= 1) {
    tg += (uint32_t)__shfl_xor((int)tg, o);
    te += (uint32_t)__shfl_xor((int)te, o);
  }
  if (lane == 0) {
    sh.wsum[wave][0] = tg;
    sh.wsum[wave][1] = te;
  }
  __syncthreads();
  uint32_t gbase = 0, ebase = 0;  // wave-uniform
  for (int i = 0; i < wave; ++i) {
    gbase += sh.wsum[i][0];
    ebase += sh.wsum[i][1];
  }
  const uint32_t n_gt = k - k_rem;
  const bool wave_ties = __ballot(eqm != 0) != 0;  // ties sit in very few waves
#pragma unroll 2
  for (int q = 0; q < EPT / 4; ++q) {
    const uint32_t ng = (uint32_t)(gtm >> (4 * q)) & 0xFu, ne = (uint32_t)(eqm >> (4 * q)) & 0xFu;
    const int pos0 = elem_pos<EPT>(wave, lane, 4 * q);
    uint64_t m[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) m[c] = __ballot((ng >> c) & 1u);
    if (m[0] | m[1] | m[2] | m[3]) {
      uint32_t r = gbase;
#pragma unroll
      for (int c = 0; c < 4; ++c) r = lanes_below(m[c], r);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((ng >> c) & 1u) emit(pos0 + c, r++);
#pragma unroll
      for (int c = 0; c < 4; ++c) gbase += (uint32_t)__builtin_popcountll(m[c]);
    }
    if (!wave_ties) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) m[c] = __ballot((ne >> c) & 1u);
    if (m[0] | m[1] | m[2] | m[3]) {
      uint32_t r = ebase;
#pragma unroll
      for (int c = 0; c < 4; ++c) r = lanes_below(m[c], r);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if ((ne >> c) & 1u) {
          if (r < k_rem) emit(pos0 + c, n_gt + r);
          ++r;
        }
#pragma unroll
      for (int c = 0; c < 4; ++c) ebase += (uint32_t)__builtin_popcountll(m[c]);
    }
  }
}

// Copy the staged index list (k <= TK_STAGE entries) to dst with 16-byte stores where aligned.
__device__ __forceinline__ void store_staged(const TopkShared& sh, int32_t* __restrict__ dst, int32_t k) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (((uintptr_t)dst & 15) == 0) {
    const int k4 = k & ~3;
    for (int i = 4 * tid; i < k4; i += 4 * TK_THREADS)
      *reinterpret_cast<v4i*>(dst + i) = *reinterpret_cast<const v4i*>(sh.stage + i);
    for (int i = k4 + tid; i < k; i += TK_THREADS) dst[i] = sh.stage[i];
  } else {
    for (int i = tid; i < k; i += TK_THREADS) dst[i] = sh.stage[i];
  }
}

// ---------------------------------------------------------------------------------------------
// Chunks of rows that span several chunks (512 threads, the chunk held in registers, 64 scores
// per thread): one read of the chunk, the sampled pivot and the candidate compaction run on the
// registers, and the candidates are written for the merge.

constexpr int TK_CAND = 4096;     // candidate keys of the sampled threshold search
constexpr int TK_CAND_EPT = TK_CAND / TK_THREADS;
constexpr int TK_MAP_WORDS = TK_CHUNK_EPT * TK_THREADS / 32;  // one bit per position of a chunk

struct TopkChunkShared : TopkShared {
  uint32_t cand[TK_CAND];
  uint32_t cpos[TK_CAND];           // position of each candidate in the chunk
  uint32_t gtmap[TK_MAP_WORDS];     // selected positions above tau
  uint32_t eqmap[TK_MAP_WORDS];     // positions equal to tau
};

// Exact threshold search over a chunk of cn > k valid elements (maximum mx, minimum mn) that
// touches most keys once (returns the number of candidates left in sh.cand / sh.cpos, or 0 when
// the select ran over all keys instead): a histogram of a 1-in-16 sample of the keys in
// equal-width value bins puts a pivot a safe margin below the expected position of the k-th
// largest key; the keys at or above the pivot are counted, and when there are between k and
// TK_CAND of them they are compacted into LDS, where the exact select finds tau and the tie
// count among them (every key >= tau is a candidate, so both are exact).  Outside that window
// (an unlucky or adversarial sample) the radix select runs over all keys.  Chunks of at most
// TK_CAND elements skip the sample.  The histogram is zero on entry and exit.
template <int EPT>
__device__ uint32_t sampled_threshold(const uint32_t (&key)[EPT], int64_t cn, uint32_t k, uint32_t mx, uint32_t mn,
                                      TopkChunkShared& sh, uint32_t& tau, uint32_t& k_rem) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (mx == mn) {
    tau = mx;
    k_rem = k;
    return 0;
  }
  uint32_t pivot = mn;  // every valid key
  if (cn > TK_CAND) {
    // sample element 17 i (i < EPT / 16) of every thread; lane l's copy sits at the lane-0 position + 4 l
    // (elem_pos), so the number of valid samples follows from cn without a reduction
    constexpr int NS = EPT / 16;  // sampled elements per thread, 17 apart
    static_assert(NS >= 1 && 17 * (NS - 1) < EPT, "sample positions");
    uint32_t smp[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) smp[i] = key[17 * i];
    uint32_t m = 0;
    for (int w = 0; w < TK_WAVES; ++w)
      for (int i = 0; i < NS; ++i) {
        const int64_t rest = cn - elem_pos<EPT>(w, 0, 17 * i);  // valid lanes: 4 l < rest
        m += (uint32_t)min<int64_t>(WAVE, max<int64_t>(0, (rest + 3) / 4));
      }
    // rank sought among the m sampled keys: the expected rank of the k-th largest key plus four
    // binomial standard deviations; none (the pivot stays mn) when the sample is too small
    const float er = (float)k * (float)m / (float)cn;
    const float w = er + 4.0f * sqrtf(er) + 16.0f;
    const float lo = key_score(mn), hi = key_score(mx);
    if (w <= (float)m && lin_range_ok(lo, hi)) {  // workgroup-uniform; mx > mn here
      // one histogram pass over the samples in LIN_BINS equal-width bins over the chunk's value
      // range: the pivot is the lower edge of the bin holding the sample of rank w, moved down by
      // more than the rounding of the bin arithmetic (a lower pivot only adds candidates)
      const float scale = (float)LIN_BINS / (hi - lo);
      int b;
      uint32_t above, cnt;
      lin_pass<NS>(smp, [](uint32_t) { return true; }, lo, scale, (uint32_t)w, sh, b, above, cnt);
      const float pf = (lo + (float)b / scale) - (fabsf(lo) * 0x1p-20f + fabsf(hi) * 0x1p-20f);
      pivot = max(score_key(pf), mn);
    }
  }
  uint32_t c = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) c += key[e] >= pivot;  // pivot >= mn >= 1: valid keys only
  // exclusive offsets of this thread's candidates
  const uint32_t incl = wave_incl_scan(c, lane);
  if (lane == 63) sh.wsum[wave][1] = incl;
  __syncthreads();
  uint32_t off = incl - c, total = 0;
  for (int i = 0; i < TK_WAVES; ++i) {
    const uint32_t w = sh.wsum[i][1];
    if (i < wave) off += w;
    total += w;
  }
  if (total < k || total > (uint32_t)TK_CAND) {  // workgroup-uniform
    radix_select<EPT>(key, k, mx, mn, sh, tau, k_rem);
    return 0;
  }
  // an opaque copy of the pivot: the counting loop's 64 compare masks are recomputed here rather
  // than kept (in scalar registers) across the scan
  uint32_t pv = __builtin_amdgcn_readfirstlane(pivot);
  asm volatile("" : "+s"(pv));
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (key[e] >= pv) {
      sh.cand[off] = key[e];
      sh.cpos[off] = (uint32_t)elem_pos<EPT>(wave, lane, e);
      ++off;
    }
  __syncthreads();
  uint32_t ck[TK_CAND_EPT];
#pragma unroll
  for (int j = 0; j < TK_CAND_EPT; ++j) {
    const uint32_t i = (uint32_t)(tid + j * TK_THREADS);
    ck[j] = i < total ? sh.cand[i] : 0u;
  }
  lin_select<TK_CAND_EPT>(ck, k, mx, pivot, sh, tau, k_rem);
  return total;
}

// Ordered emission from the candidate list (every selected element is a candidate): each
// candidate above tau sets its position's bit in one LDS bitmap, each equal to tau in another;
// thread t then owns positions 64 t .. 64 t + 63 (two words of each map), and one block scan of
// its two bit counts (packed in one word) gives its output offsets: every position above tau in
// ascending order, then the first k_rem positions equal to tau.  The maps are zero on entry.
template <typename Emit>
__device__ void emit_candidates(TopkChunkShared& sh, uint32_t total, uint32_t tau, uint32_t k, uint32_t k_rem,
                                Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (uint32_t i = (uint32_t)tid; i < total; i += TK_THREADS) {
    const uint32_t kk = sh.cand[i], p = sh.cpos[i];
    if (kk > tau)
      atomicOr(&sh.gtmap[p >> 5], 1u << (p & 31));
    else if (kk == tau)
      atomicOr(&sh.eqmap[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  static_assert(TK_MAP_WORDS == 2 * TK_THREADS, "two map words per thread");
  uint32_t g0 = sh.gtmap[2 * tid], g1 = sh.gtmap[2 * tid + 1];
  uint32_t e0 = sh.eqmap[2 * tid], e1 = sh.eqmap[2 * tid + 1];
  const uint32_t cnt = (uint32_t)(__popc(g0) + __popc(g1)) | ((uint32_t)(__popc(e0) + __popc(e1)) << 16);
  const uint32_t incl = wave_incl_scan(cnt, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();
  uint32_t off = incl - cnt;
  for (int i = 0; i < wave; ++i) off += sh.wsum[i][0];
  uint32_t go = off & 0xFFFFu, eo = off >> 16;
  const int base = 64 * tid;
  for (; g0; g0 &= g0 - 1) emit(base + __builtin_ctz(g0), go++);
  for (; g1; g1 &= g1 - 1) emit(base + 32 + __builtin_ctz(g1), go++);
  const uint32_t n_gt = k - k_rem;
  for (; e0 && eo < k_rem; e0 &= e0 - 1) emit(base + __builtin_ctz(e0), n_gt + eo++);
  for (; e1 && eo < k_rem; e1 &= e1 - 1) emit(base + 32 + __builtin_ctz(e1), n_gt + eo++);
}

// Load this thread's elements of scores[0 .. n) (1 <= n <= 512 * EPT) as keys (0 past n).  The
// loads are unconditional so that all of them are in flight before the first one is waited for:
// a group of four past the end re-reads the row's last aligned group, which is in bounds because
// rows start 16-byte aligned and their stride is a multiple of four floats.
template <int EPT>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int64_t n, uint32_t (&key)[EPT]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int last = (int)(((n + 3) & ~(int64_t)3) - 4);
  v4f v[EPT / 4];
#pragma unroll
  for (int q = 0; q < EPT / 4; ++q)
    v[q] = *reinterpret_cast<const v4f*>(row + min(elem_pos<EPT>(wave, lane, 4 * q), last));
#pragma unroll
  for (int q = 0; q < EPT / 4; ++q) {
    const int p = elem_pos<EPT>(wave, lane, 4 * q);
#pragma unroll
    for (int c = 0; c < 4; ++c) key[4 * q + c] = p + c < n ? score_key(v[q][c]) : 0u;
  }
}

// The selection of one chunk of cn (k < cn <= 512 EPT) elements with EPT elements per thread.
template <int EPT>
__device__ __forceinline__ void chunk_select(const float* __restrict__ logits, int64_t ld, int64_t t, int chunk,
                                             int64_t c0, int64_t cn, bool single, int32_t k,
                                             int32_t* __restrict__ out_idx, uint32_t* __restrict__ cand_key,
                                             int32_t* __restrict__ cand_idx, int32_t G, TopkChunkShared& sh) {
  uint32_t key[EPT];
  hist_clear(sh);
  for (int i = threadIdx.x; i < TK_MAP_WORDS; i += TK_THREADS) {
    sh.gtmap[i] = 0;
    sh.eqmap[i] = 0;
  }
  load_keys<EPT>(logits + t * ld + c0, cn, key);
  uint32_t mx, mn, tau, k_rem;
  block_minmax<EPT>(key, sh, mx, mn);
  const uint32_t ncand = sampled_threshold<EPT>(key, cn, (uint32_t)k, mx, mn, sh, tau, k_rem);
  // emission from the candidates when they hold the selection, else from the registers
  auto emit = [&](auto&& f) {
    if (ncand)
      emit_candidates(sh, ncand, tau, (uint32_t)k, k_rem, f);
    else
      emit_selected<EPT>(key, tau, (uint32_t)k, k_rem, sh, f);
  };
  if (single) {
    if (k <= TK_STAGE) {
      emit([&](int pos, uint32_t slot) { sh.stage[slot] = (int32_t)(c0 + pos); });
      store_staged(sh, out_idx, k);
    } else {
      emit([&](int pos, uint32_t slot) { out_idx[slot] = (int32_t)(c0 + pos); });
    }
  } else {
    uint32_t* ck = cand_key + (t * G + chunk) * (int64_t)k;
    int32_t* ci = cand_idx + (t * G + chunk) * (int64_t)k;
    const float* row = logits + t * ld + c0;
    emit([&](int pos, uint32_t slot) {
      ck[slot] = score_key(row[pos]);  // re-read (L2): keeps the key array out of the loop
      ci[slot] = (int32_t)(c0 + pos);
    });
  }
}

// One chunk of a row when rows may span several chunks: the chunk's candidates go to cand_key /
// cand_idx [rows][G][k] (key 0 = empty slot); rows of one chunk write their final list.
// Prefill rows: n_t = min(S, q_start + t + 1); decode rows (seq_lens given): n = seq_lens[t].
__global__ __launch_bounds__(TK_THREADS) __attribute__((amdgpu_waves_per_eu(4, 4))) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t ld, int64_t T, int64_t S, int64_t q_start,
    const int32_t* __restrict__ seq_lens, int32_t k, int32_t* __restrict__ indices,
    uint32_t* __restrict__ cand_key, int32_t* __restrict__ cand_idx, int32_t G) {
  __shared__ TopkChunkShared sh;
  const int64_t t = blockIdx.x;  // rows on x: up to 2^31 - 1 of them in one launch
  const int chunk = blockIdx.y;
  const int64_t n = seq_lens ? min((int64_t)max(seq_lens[t], 0), S) : min(S, q_start + t + 1);
  const int64_t c0 = (int64_t)chunk * TK_CHUNK;
  if (c0 >= n && chunk > 0) return;
  const int64_t cn = min(n - c0, TK_CHUNK);  // elements of this chunk
  const bool single = n <= TK_CHUNK;
  const int tid = threadIdx.x;
  int32_t* out_idx = indices + t * k;

  if (cn <= k) {  // everything in the chunk is selected
    for (int64_t i = tid; i < k; i += TK_THREADS) {
      if (single) {
        out_idx[i] = i < cn ? (int32_t)(c0 + i) : -1;
      } else {
        cand_key[(t * G + chunk) * (int64_t)k + i] = i < cn ? score_key(logits[t * ld + c0 + i]) : 0u;
        cand_idx[(t * G + chunk) * (int64_t)k + i] = i < cn ? (int32_t)(c0 + i) : -1;
      }
    }
    return;
  }
  // the narrowest register layout that holds the chunk: the work per row follows its length
  if (cn <= TK_CHUNK / 4)
    chunk_select<TK_CHUNK_EPT / 4>(logits, ld, t, chunk, c0, cn, single, k, out_idx, cand_key, cand_idx, G, sh);
  else if (cn <= TK_CHUNK / 2)
    chunk_select<TK_CHUNK_EPT / 2>(logits, ld, t, chunk, c0, cn, single, k, out_idx, cand_key, cand_idx, G, sh);
  else
    chunk_select<TK_CHUNK_EPT>(logits, ld, t, chunk, c0, cn, single, k, out_idx, cand_key, cand_idx, G, sh);
}

// ---------------------------------------------------------------------------------------------
// Whole rows of at most one chunk (256 threads; the row streamed, see the header).
constexpr int TS_THREADS = 256;
constexpr int TS_WAVES = TS_THREADS / WAVE;
constexpr int TS_BPT = TK_BINS / TS_THREADS;          // histogram bins per thread in the suffix scan
constexpr int TS_UNITS = (int)(TK_CHUNK / 4);          // 16-byte units of a full chunk
constexpr int TS_UPT = TS_UNITS / TS_THREADS;          // units per thread (32)
constexpr int TS_BATCH = 8;                            // units in flight per thread
constexpr int TS_SPT = TS_UPT / 4;                     // samples per thread (8: two from each of four units)
constexpr int TS_SAMPLES = TS_THREADS * TS_SPT;        // 2048
constexpr int TS_CAND = 4096;                          // candidate capacity
constexpr int TS_CPT = TS_CAND / TS_THREADS;           // candidate slots per thread (16)
constexpr int TS_MAP_WORDS = (int)(TK_CHUNK / 32);     // one bit per position of a chunk
constexpr int TS_MPT = TS_MAP_WORDS / TS_THREADS;      // map words per thread (4)
static_assert(TS_UPT % TS_BATCH == 0 && TS_MPT == 4, "chunk geometry");

struct TsShared {
  union {                                        // the histogram is zero whenever a select ends,
    uint32_t hist[TK_BINS];                      // so the bitmaps that reuse it start cleared
    struct {
      uint32_t gt[TS_MAP_WORDS];                 // positions above tau
      uint32_t eq[TS_MAP_WORDS];                 // positions equal to tau
    } map;
  } h;
  union {
    uint32_t samples[TS_SAMPLES];                // sample keys (0: none)
    uint16_t cand[TS_CAND];                      // candidate positions in the chunk
    int32_t stage[TK_STAGE];                     // the staged index list
  } u;
  uint32_t wsum[TS_WAVES][2];
  uint32_t red[TS_WAVES][3];
  uint32_t sel_bin, sel_above, sel_cnt;
  uint32_t small[WAVE];
  uint32_t small_n;
  uint32_t ccount;                               // candidates appended
};
static_assert(2 * TS_MAP_WORDS <= TK_BINS, "the bitmaps fit the histogram");


// Block-wide (max, min - 1, sum) of per-thread values (max 0 / min - 1 0xFFFFFFFF: nothing).
__device__ __forceinline__ void ts_block_reduce(uint32_t& mx, uint32_t& mnm1, uint32_t& sum, TsShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  mx = wave_max_u32(mx);
  mnm1 = wave_min_u32(mnm1);
  for (int o = 32; o > 0; o >>= 1) sum += (uint32_t)__shfl_xor((int)sum, o);
  if (lane == 0) {
    sh.red[wave][0] = mx;
    sh.red[wave][1] = mnm1;
    sh.red[wave][2] = sum;
  }
  __syncthreads();
  mx = 0;
  mnm1 = 0xFFFFFFFFu;
  sum = 0;
  for (int i = 0; i < TS_WAVES; ++i) {
    mx = max(mx, sh.red[i][0]);
    mnm1 = min(mnm1, sh.red[i][1]);
    sum += sh.red[i][2];
  }
}

// One histogram pass over the keys visit() produces (0 = none): as hist_pass, for 256 threads.
// The histogram is zero on entry and on exit; need must lie in 1 .. (matching keys).
template <typename Visit>
__device__ void ts_hist_pass(Visit visit, int shift, int bits, uint32_t prefix, TsShared& sh, uint32_t need,
                             uint32_t& bin, uint32_t& above_out, uint32_t& cnt_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi_shift = shift + bits;
  const uint32_t dmask = (1u << bits) - 1u;
  visit([&](uint32_t kk) {
    const bool match = kk != 0 && (hi_shift >= 32 ? true : ((kk >> hi_shift) == prefix));
    if (match) atomicAdd(&sh.h.hist[(kk >> shift) & dmask], 1u);
  });
  __syncthreads();
  // suffix counts: thread t owns the bins TS_BPT (255 - t) .. + TS_BPT - 1 (highest bins first)
  const int b0 = TS_BPT * (TS_THREADS - 1 - tid);
  uint32_t h[TS_BPT];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < TS_BPT; ++i) {
    h[i] = sh.h.hist[b0 + i];
    sh.h.hist[b0 + i] = 0;
    own += h[i];
  }
  const uint32_t incl = wave_incl_scan(own, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();
  uint32_t above = incl - own;
  for (int i = 0; i < wave; ++i) above += sh.wsum[i][0];
  if (above < need && need <= above + own) {
    uint32_t a = above;
    for (int i = TS_BPT - 1; i >= 0; --i) {
      if (need <= a + h[i]) {
        sh.sel_bin = (uint32_t)(b0 + i);
        sh.sel_above = a;
        sh.sel_cnt = h[i];
        break;
      }
      a += h[i];
    }
  }
  __syncthreads();
  bin = sh.sel_bin;
  above_out = sh.sel_above;
  cnt_out = sh.sel_cnt;
}

// The end of an exact select once the bin holding the sought rank has cnt <= 64 keys: as
// small_finish.  sh.small_n is zero on entry and on exit.
template <typename Visit, typename Match>
__device__ void ts_small_finish_if(Visit visit, Match match, uint32_t cnt, uint32_t need, TsShared& sh,
                                   uint32_t& tau, uint32_t& k_rem) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  visit([&](uint32_t kk) {
    if (kk != 0 && match(kk)) sh.small[atomicAdd(&sh.small_n, 1u)] = kk;
  });
  __syncthreads();
  if (wave == 0) {
    const uint32_t x = (uint32_t)lane < cnt ? sh.small[lane] : 0u;
    uint32_t gt = 0, eq = 0;
    const uint32_t cu = (uint32_t)__builtin_amdgcn_readfirstlane((int)cnt);  // workgroup-uniform
    for (uint32_t m = 0; m < cu; ++m) {
      const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, (int)m);  // lane m holds small[m]
      gt += y > x;
      eq += y == x;
    }
    if ((uint32_t)lane < cnt && gt < need && need <= gt + eq) {  // every copy of tau writes the same
      sh.sel_bin = x;
      sh.sel_above = need - gt;
    }
    if (lane == 0) sh.small_n = 0;
  }
  __syncthreads();
  tau = sh.sel_bin;
  k_rem = sh.sel_above;
}

template <typename Visit>
__device__ void ts_small_finish(Visit visit, int shift, uint32_t prefix, uint32_t cnt, uint32_t need, TsShared& sh,
                                uint32_t& tau, uint32_t& k_rem) {
  ts_small_finish_if(visit, [&](uint32_t kk) { return (kk >> shift) == prefix; }, cnt, need, sh, tau, k_rem);
}

constexpr int TS_LPT = LIN_BINS / TS_THREADS;  // bins per thread in the suffix scan

// One histogram pass over the scores of the keys visit() produces (0 = none) that match(), in
// LIN_BINS bins of width 1 / scale from lo (lo and scale finite): the bin holding the need-th
// largest of them (1 <= need <= their count), the matching keys above it and in it.  The
// histogram is zero on entry and on exit.
template <typename Visit, typename Match>
__device__ void ts_lin_pass(Visit visit, Match match, float lo, float scale, uint32_t need, TsShared& sh, int& bin,
                            uint32_t& above_out, uint32_t& cnt_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  visit([&](uint32_t kk) {
    if (kk != 0 && match(kk)) atomicAdd(&sh.h.hist[lin_bin(key_score(kk), lo, scale)], 1u);
  });
  __syncthreads();
  // thread t owns bins TS_LPT (255 - t) .. + TS_LPT - 1: the highest bins first
  const int b0 = TS_LPT * (TS_THREADS - 1 - tid);
  uint32_t h[TS_LPT];
  uint32_t own = 0;
#pragma unroll
  for (int i = 0; i < TS_LPT; ++i) {
    h[i] = sh.h.hist[b0 + i];
    sh.h.hist[b0 + i] = 0;
    own += h[i];
  }
  const uint32_t incl = wave_incl_scan(own, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();
  uint32_t above = incl - own;
  for (int i = 0; i < wave; ++i) above += sh.wsum[i][0];
  if (above < need && need <= above + own) {
    uint32_t a = above;
    for (int i = TS_LPT - 1; i >= 0; --i) {
      if (need <= a + h[i]) {
        sh.sel_bin = (uint32_t)(b0 + i);
        sh.sel_above = a;
        sh.sel_cnt = h[i];
        break;
      }
      a += h[i];
    }
  }
  __syncthreads();
  bin = (int)sh.sel_bin;
  above_out = sh.sel_above;
  cnt_out = sh.sel_cnt;
}

// Exact select over the keys visit() produces: tau (the k-th largest) and k_rem (how many keys
// equal to tau are taken).  mx, mn: maximum and a lower bound >= 1 of the valid keys.  Requires at
// least k valid keys and a zero histogram.
template <typename Visit>
__device__ void ts_radix_select(Visit visit, uint32_t k, uint32_t mx, uint32_t mn, TsShared& sh, uint32_t& tau,
                                uint32_t& k_rem) {
  if (mx == mn) {
    tau = mx;
    k_rem = k;
    return;
  }
  const int hb = 31 - __clz(mx ^ mn);
  int shift = hb >= TK_DIGIT - 1 ? hb - (TK_DIGIT - 1) : 0;
  int bits = hb - shift + 1;
  uint32_t prefix = (hb == 31) ? 0u : (mx >> (hb + 1));
  uint32_t need = k;
  while (true) {
    uint32_t bin, above, cnt;
    ts_hist_pass(visit, shift, bits, prefix, sh, need, bin, above, cnt);
    need -= above;
    prefix = (shift + bits >= 32 ? 0u : (prefix << bits)) | bin;
    if (shift == 0) break;
    if (cnt <= (uint32_t)WAVE) {  // workgroup-uniform
      ts_small_finish(visit, shift, prefix, cnt, need, sh, tau, k_rem);
      return;
    }
    bits = shift >= TK_DIGIT ? TK_DIGIT : shift;
    shift -= bits;
  }
  tau = prefix;
  k_rem = need;
}

// Ordered emission from the bitmaps: thread t owns positions 128 t .. 128 t + 127 (four words of
// each map); one block scan of its two bit counts (packed in one word) gives the output slots:
// every position above tau in ascending order, then the first k_rem positions equal to tau.
template <typename Emit>
__device__ void ts_emit_maps(TsShared& sh, uint32_t k, uint32_t k_rem, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t g[TS_MPT], e[TS_MPT];
  uint32_t ng = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < TS_MPT; ++i) {
    g[i] = sh.h.map.gt[TS_MPT * tid + i];
    e[i] = sh.h.map.eq[TS_MPT * tid + i];
    ng += (uint32_t)__popc(g[i]);
    ne += (uint32_t)__popc(e[i]);
  }
  const uint32_t cnt = ng | (ne << 16);
  const uint32_t incl = wave_incl_scan(cnt, lane);
  if (lane == 63) sh.wsum[wave][0] = incl;
  __syncthreads();  // also: every bitmap word read before the staged list may overwrite LDS
  uint32_t off = incl - cnt;
  for (int i = 0; i < wave; ++i) off += sh.wsum[i][0];
  uint32_t go = off & 0xFFFFu, eo = off >> 16;
  const uint32_t n_gt = k - k_rem;
  const int base = 128 * tid;
#pragma unroll
  for (int i = 0; i < TS_MPT; ++i)
    for (uint32_t m = g[i]; m; m &= m - 1) emit(base + 32 * i + __builtin_ctz(m), go++);
#pragma unroll
  for (int i = 0; i < TS_MPT; ++i)
    for (uint32_t m = e[i]; m && eo < k_rem; m &= m - 1) emit(base + 32 * i + __builtin_ctz(m), n_gt + eo++);
}

// The selection of one chunk of cn (k < cn <= 32768) scores at row (row + 16-byte aligned).
template <typename Emit>
__device__ void ts_chunk_select(const float* __restrict__ row, int cn, uint32_t k, TsShared& sh, Emit emit) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const v4f* row4 = reinterpret_cast<const v4f*>(row);
  const int nunits = (cn + 3) >> 2;
  const int last = nunits - 1;
  // every key of the chunk (0 past cn), streamed in batches of TS_BATCH units per thread; a unit
  // past the end re-reads the last one (in bounds: rows are 16-byte aligned, their stride a
  // multiple of four floats)
  auto stream_keys = [&](auto&& f) {
    for (int j0 = 0; j0 * TS_THREADS < nunits; j0 += TS_BATCH) {  // workgroup-uniform
      v4f v[TS_BATCH];
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b) v[b] = row4[min(tid + TS_THREADS * (j0 + b), last)];
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b) {
        const int p0 = 4 * (tid + TS_THREADS * (j0 + b));
#pragma unroll
        for (int c = 0; c < 4; ++c) f(p0 + c < cn ? score_key(v[b][c]) : 0u);
      }
    }
  };

  // ---- 1. the pivot: every element when the row is small, else a value histogram of samples
  float pf = -__builtin_inff();
  if (cn > TS_CAND) {
    // sampled units: thread t of wave w reads units t + 256 j for j = w, w + 8, ... (an eighth of
    // the chunk, in 1 KB blocks), samples = the unit's first two scores
    uint32_t smx = 0, smnm1 = 0xFFFFFFFFu, m = 0;
    {
      v4f v[TS_SPT / 2];
#pragma unroll
      for (int i = 0; i < TS_SPT / 2; ++i) v[i] = row4[min(tid + TS_THREADS * (wave + 8 * i), last)];
#pragma unroll
      for (int i = 0; i < TS_SPT; ++i) {
        const int p = 4 * (tid + TS_THREADS * (wave + 8 * (i >> 1))) + (i & 1);
        const uint32_t kk = p < cn ? score_key(v[i >> 1][i & 1]) : 0u;
        sh.u.samples[tid + TS_THREADS * i] = kk;
        smx = max(smx, kk);
        smnm1 = min(smnm1, kk - 1u);
        m += kk != 0;
      }
    }
    ts_block_reduce(smx, smnm1, m, sh);  // its barrier also publishes the samples
    // rank sought among the m samples: the expected rank of the k-th largest score plus four
    // binomial standard deviations; none (the pivot stays -inf) when the sample is too small
    const float er = (float)k * (float)m / (float)cn;
    const float w = er + 4.0f * sqrtf(er) + 16.0f;
    if (w <= (float)m && smx != smnm1 + 1u) {
      auto visit_samples = [&](auto&& f) {
#pragma unroll
        for (int i = 0; i < TS_SPT; ++i) f(sh.u.samples[tid + TS_THREADS * i]);
      };
      // one histogram pass over the samples in LIN_BINS bins of equal width over their value
      // range: the pivot is the lower edge of the bin holding the sample of rank w, moved down by
      // more than the rounding of the bin arithmetic (a lower pivot only adds candidates)
      const float lo = key_score(smnm1 + 1u), hi = key_score(smx);
      const float range = hi - lo;
      if (lin_range_ok(lo, hi)) {  // workgroup-uniform
        const float scale = (float)LIN_BINS / range;
        int b;
        uint32_t above, cnt;
        ts_lin_pass(visit_samples, [](uint32_t) { return true; }, lo, scale, (uint32_t)w, sh, b, above, cnt);
        pf = (lo + (float)b / scale) - (fabsf(lo) * 0x1p-20f + fabsf(hi) * 0x1p-20f);
      }
    }
  }
  // ---- 2. the candidates: the positions of every score >= pf (NaN-free comparison of floats;
  // the key order is the float order with -0 == +0), appended in batches with one LDS atomic per
  // wave; a lane visits only its selected bits, so the append costs follow the candidates, not
  // the chunk
  const float pv = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(pf)));
  if (tid == 0) sh.ccount = 0;
  __syncthreads();  // also: every sample read before the candidate list overwrites them
  for (int j0 = 0; j0 * TS_THREADS < nunits; j0 += TS_BATCH) {  // workgroup-uniform
    v4f v[TS_BATCH];
#pragma unroll
    for (int b = 0; b < TS_BATCH; ++b) v[b] = row4[min(tid + TS_THREADS * (j0 + b), last)];
    uint32_t selm = 0;  // bit 4 b + c: unit b, score c selected
    if (4 * TS_THREADS * (j0 + TS_BATCH) <= cn) {  // every position of the batch visible
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) selm |= (uint32_t)(v[b][c] >= pv) << (4 * b + c);
    } else {
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b) {
        const int p0 = 4 * (tid + TS_THREADS * (j0 + b));
#pragma unroll
        for (int c = 0; c < 4; ++c) selm |= (uint32_t)(p0 + c < cn && v[b][c] >= pv) << (4 * b + c);
      }
    }
    const uint32_t nsel = (uint32_t)__popc(selm);
    const uint32_t incl = wave_incl_scan(nsel, lane);
    uint32_t base = 0;
    if (lane == 63 && incl) base = atomicAdd(&sh.ccount, incl);
    base = (uint32_t)__shfl((int)base, 63) + incl - nsel;
    const int pbase = 4 * (tid + TS_THREADS * j0);
    for (uint32_t m = selm; m; m &= m - 1) {
      const int e = __builtin_ctz(m);
      if (base < (uint32_t)TS_CAND) sh.u.cand[base] = (uint16_t)(pbase + 4 * TS_THREADS * (e >> 2) + (e & 3));
      ++base;
    }
  }
  __syncthreads();
  const uint32_t total = sh.ccount;
  uint32_t tau, k_rem;
  if (total >= k && total <= (uint32_t)TS_CAND) {  // workgroup-uniform
    // ---- 3. exact select over the candidates (slot tid + 256 j of this thread)
    uint32_t ck[TS_CPT], cp[TS_CPT];
    uint32_t cmx = 0, cmnm1 = 0xFFFFFFFFu, dummy = 0;
#pragma unroll
    for (int j = 0; j < TS_CPT; ++j) {
      const uint32_t i = (uint32_t)(tid + TS_THREADS * j);
      cp[j] = i < total ? sh.u.cand[i] : 0u;
    }
    float cv[TS_CPT];
#pragma unroll
    for (int j = 0; j < TS_CPT; ++j) cv[j] = row[cp[j]];  // scores re-read (cache), all in flight
#pragma unroll
    for (int j = 0; j < TS_CPT; ++j) {
      const uint32_t i = (uint32_t)(tid + TS_THREADS * j);
      ck[j] = i < total ? score_key(cv[j]) : 0u;
      cmx = max(cmx, ck[j]);
      cmnm1 = min(cmnm1, ck[j] - 1u);
    }
    ts_block_reduce(cmx, cmnm1, dummy, sh);
    auto visit_cand = [&](auto&& f) {
#pragma unroll
      for (int j = 0; j < TS_CPT; ++j) f(ck[j]);
    };
    // LIN_BINS bins of equal width over the candidates' value range, and when the bin holding the
    // k-th largest has more than 64 candidates, LIN_BINS sub-bins of that bin; one wave then ranks
    // the (at most 64) candidates of the final bin exactly.  Heavier ties: the radix select over
    // the keys.
    const uint32_t cmn = cmnm1 + 1u;
    const float lo = key_score(cmn), hi = key_score(cmx);
    bool done = false;
    if (cmx != cmn && lin_range_ok(lo, hi)) {  // workgroup-uniform
      const float scale = (float)LIN_BINS / (hi - lo);
      int b;
      uint32_t above, cnt;
      ts_lin_pass(visit_cand, [](uint32_t) { return true; }, lo, scale, k, sh, b, above, cnt);
      auto in_b = [&](uint32_t kk) { return lin_bin(key_score(kk), lo, scale) == b; };
      if (cnt <= (uint32_t)WAVE) {
        ts_small_finish_if(visit_cand, in_b, cnt, k - above, sh, tau, k_rem);
        done = true;
      } else {
        const float lo2 = lo + (float)b / scale, scale2 = scale * (float)LIN_BINS;
        int b2;
        uint32_t above2, cnt2;
        ts_lin_pass(visit_cand, in_b, lo2, scale2, k - above, sh, b2, above2, cnt2);
        if (cnt2 <= (uint32_t)WAVE) {
          ts_small_finish_if(
              visit_cand, [&](uint32_t kk) { return in_b(kk) && lin_bin(key_score(kk), lo2, scale2) == b2; }, cnt2,
              k - above - above2, sh, tau, k_rem);
          done = true;
        }
      }
    }
    if (!done) ts_radix_select(visit_cand, k, cmx, cmn, sh, tau, k_rem);
    // ---- 4. the bitmaps from the candidates (the histogram is zero after the select)
#pragma unroll
    for (int j = 0; j < TS_CPT; ++j) {
      const uint32_t kk = ck[j], p = cp[j];
      if (kk > tau)
        atomicOr(&sh.h.map.gt[p >> 5], 1u << (p & 31));
      else if (kk == tau && kk != 0)
        atomicOr(&sh.h.map.eq[p >> 5], 1u << (p & 31));
    }
  } else {
    // the candidates do not hold the selection: select and bitmaps over the whole chunk
    uint32_t mx = 0, mnm1 = 0xFFFFFFFFu, dummy = 0;
    stream_keys([&](uint32_t kk) {
      mx = max(mx, kk);
      mnm1 = min(mnm1, kk - 1u);
    });
    ts_block_reduce(mx, mnm1, dummy, sh);
    ts_radix_select(stream_keys, k, mx, mnm1 + 1u, sh, tau, k_rem);
    for (int j0 = 0; j0 * TS_THREADS < nunits; j0 += TS_BATCH) {
      v4f v[TS_BATCH];
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b) v[b] = row4[min(tid + TS_THREADS * (j0 + b), last)];
#pragma unroll
      for (int b = 0; b < TS_BATCH; ++b) {
        const int p0 = 4 * (tid + TS_THREADS * (j0 + b));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t pp = (uint32_t)(p0 + c);
          const uint32_t kk = p0 + c < cn ? score_key(v[b][c]) : 0u;
          if (kk > tau)
            atomicOr(&sh.h.map.gt[pp >> 5], 1u << (pp & 31));
          else if (kk == tau && kk != 0)
            atomicOr(&sh.h.map.eq[pp >> 5], 1u << (pp & 31));
        }
      }
    }
  }
  __syncthreads();
  ts_emit_maps(sh, k, k_rem, emit);
}

// Copy the staged index list (k <= TK_STAGE entries) to dst (256 threads).
__device__ __forceinline__ void ts_store_staged(const TsShared& sh, int32_t* __restrict__ dst, int32_t k) {
  __syncthreads();
  const int tid = threadIdx.x;
  if (((uintptr_t)dst & 15) == 0) {
    const int k4 = k & ~3;
    for (int i = 4 * tid; i < k4; i += 4 * TS_THREADS)
      *reinterpret_cast<v4i*>(dst + i) = *reinterpret_cast<const v4i*>(sh.u.stage + i);
    for (int i = k4 + tid; i < k; i += TS_THREADS) dst[i] = sh.u.stage[i];
  } else {
    for (int i = tid; i < k; i += TS_THREADS) dst[i] = sh.u.stage[i];
  }
}

// One whole row (every row fits one chunk): its final index list.
// Prefill rows: n_t = min(S, q_start + t + 1); decode rows (seq_lens given): n = seq_lens[t].
__global__ __launch_bounds__(TS_THREADS) void topk_row_kernel(
    const float* __restrict__ logits, int64_t ld, int64_t S, int64_t q_start,
    const int32_t* __restrict__ seq_lens, int32_t k, int32_t* __restrict__ indices) {
  __shared__ TsShared sh;
  const int64_t t = blockIdx.x;  // rows on x: up to 2^31 - 1 of them in one launch
  const int64_t n = seq_lens ? min((int64_t)max(seq_lens[t], 0), S) : min(S, q_start + t + 1);
  const int tid = threadIdx.x;
  int32_t* out_idx = indices + t * k;
  if (n <= k) {  // everything visible is selected
    for (int64_t i = tid; i < k; i += TS_THREADS) out_idx[i] = i < n ? (int32_t)i : -1;
    return;
  }
  for (int i = tid; i < TK_BINS; i += TS_THREADS) sh.h.hist[i] = 0;
  if (tid == 0) sh.small_n = 0;
  const float* row = logits + t * ld;
  const bool staged = k <= TK_STAGE;  // the list staged in LDS, else written straight out
  ts_chunk_select(row, (int)n, (uint32_t)k, sh, [&](int pos, uint32_t slot) {
    if (staged)
      sh.u.stage[slot] = pos;
    else
      out_idx[slot] = pos;
  });
  if (staged) ts_store_staged(sh, out_idx, k);
}

// Merge the chunk candidates of rows with more than one chunk.
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    int64_t T, int64_t S, int64_t q_start, const int32_t* __restrict__ seq_lens, int32_t k,
    int32_t* __restrict__ indices, const uint32_t* __restrict__ cand_key,
    const int32_t* __restrict__ cand_idx, int32_t G) {
  __shared__ TopkShared sh;
  const int64_t t = blockIdx.x;
  const int64_t n = seq_lens ? min((int64_t)max(seq_lens[t], 0), S) : min(S, q_start + t + 1);
  if (n <= TK_CHUNK) return;  // finished by the chunk kernel
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = (int)((n + TK_CHUNK - 1) / TK_CHUNK);
  const int64_t total = (int64_t)nch * k;  // <= 512 * TK_MERGE_EPT (checked on the host)
  const uint32_t* ck = cand_key + t * G * (int64_t)k;
  const int32_t* ci = cand_idx + t * G * (int64_t)k;
  uint32_t key[TK_MERGE_EPT];
  hist_clear(sh);
  uint32_t raw[TK_MERGE_EPT];
#pragma unroll
  for (int e = 0; e < TK_MERGE_EPT; ++e)  // unconditional loads (clamped index), masked below
    raw[e] = ck[min<int64_t>(elem_pos<TK_MERGE_EPT>(wave, lane, e), total - 1)];
#pragma unroll
  for (int e = 0; e < TK_MERGE_EPT; ++e) key[e] = elem_pos<TK_MERGE_EPT>(wave, lane, e) < total ? raw[e] : 0u;
  uint32_t mx, mn, tau, k_rem;
  block_minmax<TK_MERGE_EPT>(key, sh, mx, mn);
  lin_select<TK_MERGE_EPT>(key, (uint32_t)k, mx, mn, sh, tau, k_rem);
  int32_t* out_idx = indices + t * k;
  if (k <= TK_STAGE) {
    emit_selected<TK_MERGE_EPT>(key, tau, (uint32_t)k, k_rem, sh,
                                [&](int pos, uint32_t slot) { sh.stage[slot] = ci[pos]; });
    store_staged(sh, out_idx, k);
  } else {
    emit_selected<TK_MERGE_EPT>(key, tau, (uint32_t)k, k_rem, sh,
                                [&](int pos, uint32_t slot) { out_idx[slot] = ci[pos]; });
  }
}

int32_t topk_chunks(int64_t S) { return (int32_t)((S + TK_CHUNK - 1) / TK_CHUNK); }

size_t topk_workspace_bytes(int64_t T, int64_t S, int32_t k) {
  const int32_t G = topk_chunks(S);
  if (G <= 1) return 0;
  return (size_t)T * G * k * (sizeof(uint32_t) + sizeof(int32_t));
}

bool topk_supported(int64_t S, int32_t k) {
  const int32_t G = topk_chunks(S);
  return k >= 1 && k <= TK_CHUNK && (G <= 1 || (int64_t)G * k <= (int64_t)TK_THREADS * TK_MERGE_EPT);
}

hipError_t launch_topk(const float* logits, int64_t ld, int64_t T, int64_t S, int64_t q_start,
                       const int32_t* seq_lens, int32_t k, int32_t* indices, void* workspace,
                       hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  const int32_t G = topk_chunks(S);
  uint32_t* ck = nullptr;
  int32_t* ci = nullptr;
  if (G > 1) {
    ck = reinterpret_cast<uint32_t*>(workspace);
    ci = reinterpret_cast<int32_t*>(ck + (size_t)T * G * k);
  }
  if (G <= 1)
    return launch("topk_row_kernel", topk_row_kernel, dim3((unsigned)T), dim3(TS_THREADS), 0, stream, logits, ld,
                  S, q_start, seq_lens, k, indices);
  const hipError_t e = launch("topk_chunk_kernel", topk_chunk_kernel, dim3((unsigned)T, (unsigned)G),
                              dim3(TK_THREADS), 0, stream, logits, ld, T, S, q_start, seq_lens, k, indices, ck, ci, G);
  if (e != hipSuccess) return e;
  return launch("topk_merge_kernel", topk_merge_kernel, dim3((unsigned)T), dim3(TK_THREADS), 0, stream, T, S,
                q_start, seq_lens, k, indices, ck, ci, G);
}

}  // namespace dsa
