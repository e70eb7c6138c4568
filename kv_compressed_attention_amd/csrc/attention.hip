// Bucket-restricted flash attention (AnnSA / AnnCA) on gfx950.
//
// o_q = sum_j softmax_j(scale * q.k_j + bias_j) v_j, where the key set of q
// is the keys of its bucket(s) (AnnSA: paperlayer.ai section 5 "AnnSA",
// gist.science AnnSA), a kept-prompt list (AnnCA), or all keys; bias_j is
// ln m_j for a TempCache group of m_j merged keys (Lemma 5.1, paperlayer.ai
// appendix A).
//
// bf16 kernel layout.  A workgroup of 4 waves owns 64 query rows, taken in
// index (bucket) order; each wave's MFMA rows are 16 of them.  The key list
// of the workgroup is the key ranges of its rows' distinct buckets (both
// probes), concatenated, and is streamed in chunks of 32 slots shared by the
// four waves; a (slot, row) score counts only where the slot lies in one of
// the row's own ranges, so small buckets share chunks.  Per chunk:
//   the chunk's 32 K and V rows and 32 biases go from HBM to LDS with the
//   16-byte direct loads (double-buffered: chunk c + 1 loads while chunk c
//   is computed), K and V rows stored with their 16-byte pieces
//   XOR-swizzled;
//   S^T[32 slots x 16 rows] = K Q^T   two groups of d/32
//                                      v_mfma_f32_16x16x32_bf16 (a chunk no
//                                      row of the wave uses is skipped; in
//                                      list and dense mode also such a half);
//   online softmax in float32 with exp2, row max shared by the 4 lanes of a
//   row;
//   O^T[d x 16 rows] += V^T P^T       d/16 MFMAs.  P^T comes out of S^T's
//                                      accumulator layout with no shuffles; V^T
//                                      comes from gfx950's transposing LDS
//                                      reads (ds_read_b64_tr_b16), two per
//                                      16-dim block.

#include "common.h"
#include "kernels.h"

namespace fastar {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Occupancy: 4 workgroups per CU, 3 with two probes (its 128-register
// budget at 4 spilled), 2 in table mode (up to 8 ranges per row).
// MODE: 0 bucket, 1 key list, 2 dense, 3 tables (several LSH tables and/or
// more than two probes: P is then the capacity of a row's (table, probe)
// list, ntab * ppt of it used).  Every head's k and v rows lie within 4 GiB
// of the head's first row (checked by the caller), so row offsets are 32-bit
// byte offsets from the head's base.
template <int D, int P, int MODE>
__global__ __launch_bounds__(256, MODE == 3 ? 2 : (P == 2 ? 3 : 4)) void attn_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t q_sh, int64_t q_st, int64_t Nq,
    const int32_t* __restrict__ q_bucket, const int32_t* __restrict__ q_perm,
    const uint16_t* __restrict__ k, int64_t k_sh, int64_t k_st,
    const uint16_t* __restrict__ v, int64_t v_sh, int64_t v_st, int64_t Nk,
    const float* __restrict__ key_bias, const int32_t* __restrict__ k_offsets,
    const int32_t* __restrict__ k_perm, int nbits, const int32_t* __restrict__ key_list,
    const int32_t* __restrict__ n_key_list, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int H, const int32_t* __restrict__ k_bucket, int ntab, int ppt,
    int32_t* __restrict__ n_att) {
  constexpr bool kList = MODE == 1 || MODE == 2;  // every row's keys are one list
  constexpr int E = MODE == 3 ? P : 1;            // (table, probe) entries of a row
  constexpr int NC = D / 32;                      // k-chunks of the QK^T contraction
  constexpr int NB = D / 16;                      // 16-dim output blocks
  constexpr int kPieces = D / 8;                  // 16-byte pieces of a row
  constexpr int kDmaRows = 64 / kPieces;          // rows one 64-lane 16-byte LDS load fills
  constexpr int kDmaPerWave = 32 / kDmaRows / 4;  // such loads per wave, tile and chunk
  // double-buffered chunk tiles, shared by the workgroup's waves: even
  // chunks in the A buffers, odd chunks in the B buffers (separate arrays,
  // so that reads of one are not held up by loads in flight to the other)
  __shared__ __attribute__((aligned(16))) uint16_t ktA[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t ktB[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vtA[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vtB[32 * D];
  __shared__ __attribute__((aligned(16))) float btA[32];
  __shared__ __attribute__((aligned(16))) float btB[32];
  // MODE 3: the chunk's keys' buckets in tables 0 .. ntab - 2 (the dedup test)
  __shared__ __attribute__((aligned(16))) int32_t kdA[MODE == 3 ? 3 * 32 : 4];
  __shared__ __attribute__((aligned(16))) int32_t kdB[MODE == 3 ? 3 * 32 : 4];
  // per wave: the key ids of the chunk after next (lane l's ids at [i][l]),
  // gathered by 4-byte direct loads so that no register load stays in
  // flight across the chunk loop (the compiler would wait for such a load
  // before the first reuse of its register, which fell before the LDS
  // reads of the current chunk and stalled them on the next chunk's rows)
  __shared__ __attribute__((aligned(16))) int32_t kid[MODE == 2 ? 1 : 4][kDmaPerWave + 1][FASTAR_WAVE];
  // logical block (64-row block, head), XCD-grouped
  const int64_t nbx = (Nq + 63) / 64;
  const int64_t lb = xcd_block(blockIdx.x, nbx * H);
  if (lb >= nbx * H) return;  // the whole workgroup
  const int h = (int)(lb / nbx);
  const int64_t R0 = (lb - (int64_t)h * nbx) * 64;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  // the chunk row this lane addresses for the V^T operand's transposing reads
  const int vrow = 4 * g + ((l >> 2) & 3);
  // this lane's MFMA row: workgroup row 16 wave + col
  const int64_t r = R0 + 16 * wave + col;
  const bool rvalid = r < Nq;
  int64_t t = 0;
  if (rvalid) t = (MODE == 0 || MODE == 3) ? (int64_t)q_perm[(int64_t)h * Nq + r] : r;
  // and its row of the workgroup's bucket table: workgroup row l
  int c0 = INT_MAX, c1 = INT_MAX;
  const bool wvalid = R0 + l < Nq;
  if (MODE == 0 && wvalid) {
    const int64_t tw = q_perm[(int64_t)h * Nq + R0 + l];
    const int32_t* qb = q_bucket + ((int64_t)h * Nq + tw) * P;
    c0 = qb[0];
    if (P == 2) c1 = qb[1];
  }
  // MODE 3: workgroup row l's entries as t << nbits | bucket (ce, INT_MAX
  // when absent; the pass loop consumes them), each entry's table (te), and
  // the MFMA row's buckets per entry (rq) for the dedup test: a key counts
  // in the first table that retains it
  int ce[E], te[E], rq[E];
  if (MODE == 3) {
    int64_t tw = 0;
    if (wvalid) tw = q_perm[(int64_t)h * Nq + R0 + l];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      te[e] = e / ppt;
      ce[e] = INT_MAX;
      rq[e] = -1;
      if (e < ntab * ppt) {
        const int64_t row0 = ((int64_t)te[e] * H + h) * Nq;
        const int pp = e - te[e] * ppt;
        if (wvalid) ce[e] = (te[e] << nbits) | (q_bucket[(row0 + tw) * ppt + pp] & ((1 << nbits) - 1));
        if (rvalid) rq[e] = q_bucket[(row0 + t) * ppt + pp];
      }
    }
  }

  // B operand of S^T = K Q^T: query row `col`, dims 32c + 8g .. +8
  bf16x8_t qop[NC];
  {
    const uint16_t* qrow = q + (int64_t)h * q_sh + t * q_st;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      if (!rvalid) u = make_uint4(0u, 0u, 0u, 0u);
      qop[c] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  float m = -INFINITY;
  float lsum = 0.f;
  f32x4_t acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const char* kh = reinterpret_cast<const char*>(k + (int64_t)h * k_sh);
  const char* vh = reinterpret_cast<const char*>(v + (int64_t)h * v_sh);
  const uint32_t kst_b = (uint32_t)(k_st * 2), vst_b = (uint32_t)(v_st * 2);
  const float* bh = key_bias ? key_bias + (int64_t)h * Nk : nullptr;
  const int32_t* idx_h = nullptr;
  if (MODE == 0) idx_h = k_perm + (int64_t)h * Nk;
  if (MODE == 1) idx_h = key_list + (int64_t)h * Nk;
  if (MODE == 3) idx_h = k_perm;  // positions include the (table, head) row
  int cnt = 0;                    // MODE 3: the row's attended keys (this lane's share)

  // Batches of passes.  With two probes a pass is one distinct bucket of the
  // workgroup's 64 rows (either probe), in ascending order, up to 64 per
  // batch (lane i holds pass i); with one probe, one per run of equal
  // buckets in row order (one per distinct bucket when the rows come in
  // bucket order; any order is still correct, as a bucket seen twice is then
  // just loaded twice); in list and dense mode one pass over the list or all
  // keys.  The batch's key list is its passes' key ranges, concatenated.
  // Every wave builds the same table, so loop counts agree across the
  // workgroup.
  while (true) {
    int npass = 0, xs = 0, pkb = 0, pke = 0, pr0 = -1, pr1 = -1;
    int pr[E];
#pragma unroll
    for (int e = 0; e < E; ++e) pr[e] = -1;
    if (MODE == 0 && P == 1) {
      // one probe: the rows come in bucket order (rows past the end hold
      // INT_MAX, last), so a pass opens wherever a row's bucket differs from
      // the previous row's, and the 64 rows' passes fit one batch
      const int cprev = __shfl(c0, l > 0 ? l - 1 : 0, FASTAR_WAVE);
      const uint64_t opens = ballot64(c0 != INT_MAX && (l == 0 || cprev != c0));
      npass = __popcll(opens);
      if (npass == 0) break;
      if (c0 != INT_MAX) pr0 = __popcll(opens & (lanemask_lt() | (1ull << l))) - 1;
      // lane p: the row that opens pass p (the (p+1)-th set bit of opens)
      int pos = 0, kth = l;
      uint64_t mk = opens;
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) {
        const int cnt = __popcll(mk & ((1ull << w) - 1ull));
        if (kth >= cnt) {
          kth -= cnt;
          mk >>= w;
          pos += w;
        }
      }
      xs = __shfl(c0, pos & (FASTAR_WAVE - 1), FASTAR_WAVE);
      c0 = INT_MAX;
      if (l < npass) {
        const int32_t* off = k_offsets + (int64_t)h * ((1 << nbits) + 1) + xs;
        pkb = off[0];
        pke = off[1];
      }
    } else if (MODE == 3) {
      // a pass per distinct (table, bucket) of the rows' entries, ascending
      while (npass < FASTAR_WAVE) {
        int mn = INT_MAX;
#pragma unroll
        for (int e = 0; e < E; ++e) mn = min(mn, ce[e]);
        const int X = wave_min_dpp(mn);
        if (X == INT_MAX) break;
        if (l == npass) xs = X;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if (ce[e] == X) {
            ce[e] = INT_MAX;
            pr[e] = npass;
          }
        ++npass;
      }
      if (npass == 0) break;
      if (l < npass) {
        // positions in the tables' perms [ntab][H][Nk]
        const int64_t hb = (int64_t)(xs >> nbits) * H + h;
        const int32_t* off = k_offsets + hb * ((1 << nbits) + 1) + (xs & ((1 << nbits) - 1));
        pkb = (int)(hb * Nk) + off[0];
        pke = (int)(hb * Nk) + off[1];
      }
    } else if (MODE == 0) {
      while (npass < FASTAR_WAVE) {
        const int X = wave_min_dpp(min(c0, c1));
        if (X == INT_MAX) break;
        if (l == npass) xs = X;
        if (c0 == X) {
          c0 = INT_MAX;
          pr0 = npass;
        }
        if (c1 == X) {
          c1 = INT_MAX;
          pr1 = npass;
        }
        ++npass;
      }
      if (npass == 0) break;
      if (l < npass) {
        const int32_t* off = k_offsets + (int64_t)h * ((1 << nbits) + 1) + xs;
        pkb = off[0];
        pke = off[1];
      }
    } else {
      npass = 1;
      int64_t ke = Nk;
      if (n_key_list) {  // list mode, or dense over a head's first n keys
        const int64_t nl = n_key_list[h];
        ke = nl < 0 ? 0 : (nl < Nk ? nl : Nk);
      }
      pke = (int)ke;
      if (wvalid) pr0 = 0;
    }
    const int len = l < npass ? pke - pkb : 0;
    // lane p < npass: pre = slots of the passes before p; workgroup row l's
    // slot ranges [lo0, lo0 + n0) and, with two probes, [lo1, lo1 + n1)
    int pre = 0, total = 0;
    uint32_t lo0 = 0u, n0 = 0u, lo1 = 0u, n1 = 0u;
    uint32_t loe[E], ne[E];
#pragma unroll
    for (int e = 0; e < E; ++e) loe[e] = ne[e] = 0u;
    if (MODE == 0 && P == 1) {
      // a prefix sum over the passes; row l's range is its pass's
      const int incl = (int)wave_incl_scan_dpp((uint32_t)len);
      pre = incl - len;
      total = __builtin_amdgcn_readlane(incl, FASTAR_WAVE - 1);
      const int pl = pr0 < 0 ? 0 : pr0;
      const int lo = __shfl(pre, pl, FASTAR_WAVE), n = __shfl(len, pl, FASTAR_WAVE);
      if (pr0 >= 0) {
        lo0 = (uint32_t)lo;
        n0 = (uint32_t)n;
      }
    } else {
      for (int p = 0; p < npass; ++p) {
        const int lp = __builtin_amdgcn_readlane(len, p);
        if (l == p) pre = total;
        if (pr0 == p) {
          lo0 = (uint32_t)total;
          n0 = (uint32_t)lp;
        }
        if (P == 2 && pr1 == p) {
          lo1 = (uint32_t)total;
          n1 = (uint32_t)lp;
        }
        if (MODE == 3) {
#pragma unroll
          for (int e = 0; e < E; ++e)
            if (pr[e] == p) {
              loe[e] = (uint32_t)total;
              ne[e] = (uint32_t)lp;
            }
        }
        total += lp;
      }
    }
    // the MFMA row's ranges
    const int src = 16 * wave + col;
    const uint32_t rlo0 = (uint32_t)__shfl((int)lo0, src, FASTAR_WAVE);
    const uint32_t rn0 = (uint32_t)__shfl((int)n0, src, FASTAR_WAVE);
    uint32_t rlo1 = 0u, rn1 = 0u;
    if (P == 2 && MODE == 0) {
      rlo1 = (uint32_t)__shfl((int)lo1, src, FASTAR_WAVE);
      rn1 = (uint32_t)__shfl((int)n1, src, FASTAR_WAVE);
    }
    uint32_t rloe[E], rne[E];
    if (MODE == 3) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        rloe[e] = (uint32_t)__shfl((int)loe[e], src, FASTAR_WAVE);
        rne[e] = (uint32_t)__shfl((int)ne[e], src, FASTAR_WAVE);
      }
    }
    // does any of the MFMA row's ranges meet slots [a, a + w)?
    auto meets = [&](uint32_t a, uint32_t w) {
      bool u = rn0 > 0u && rlo0 < a + w && rlo0 + rn0 > a;
      if (P == 2 && MODE == 0) u = u || (rn1 > 0u && rlo1 < a + w && rlo1 + rn1 > a);
      if (MODE == 3) {
#pragma unroll
        for (int e = 0; e < E; ++e) u = u || (rne[e] > 0u && rloe[e] < a + w && rloe[e] + rne[e] > a);
      }
      return u;
    };
    const int kb_pre = pkb - pre;  // slot j of pass p is position j + kb_pre_p
    const bool is_pass = l < npass;
    // positions (in the index's permutation) of the keys this lane loads
    // for chunk c: the rows of its 16-byte loads, then (lanes < 8) the bias
    // of chunk row 8 wave + l
    auto chunk_pos = [&](int c, int* key) {
      const int j0 = 32 * c, j1 = min(32 * c + 31, total - 1);
      // the passes that chunk c overlaps: pa .. pb
      const int pa = __popcll(ballot64(is_pass && pre <= j0)) - 1;
      const int pb = __popcll(ballot64(is_pass && pre <= j1)) - 1;
      const int base_a = __builtin_amdgcn_readlane(kb_pre, pa);
      int j[kDmaPerWave + 1], base[kDmaPerWave + 1];
#pragma unroll
      for (int i = 0; i <= kDmaPerWave; ++i) {
        const int row = i < kDmaPerWave ? (wave * kDmaPerWave + i) * kDmaRows + l / kPieces
                                        : 8 * wave + (l & 7);
        j[i] = min(j0 + row, total - 1);  // past the end: a loaded, unused key
        base[i] = base_a;
      }
      // one walk over the passes for all of the lane's keys (selects, no branches)
      for (int p = pa + 1; p <= pb; ++p) {
        const int pre_p = __builtin_amdgcn_readlane(pre, p);
        const int kb_p = __builtin_amdgcn_readlane(kb_pre, p);
#pragma unroll
        for (int i = 0; i <= kDmaPerWave; ++i) base[i] = pre_p <= j[i] ? kb_p : base[i];
      }
#pragma unroll
      for (int i = 0; i <= kDmaPerWave; ++i) key[i] = j[i] + base[i];
    };
    // the keys themselves, now (dense mode: the positions are the keys)
    auto chunk_keys = [&](int c, int* key) {
      chunk_pos(c, key);
      if (MODE != 2) {
#pragma unroll
        for (int i = 0; i <= kDmaPerWave; ++i) key[i] = idx_h[key[i]];
      }
    };
    // ... or requested into this wave's kid slots, to be read after the next
    // wait for all of the wave's loads
    auto chunk_keys_async = [&](int c, int* key) {
      if constexpr (MODE == 2) {
        chunk_pos(c, key);
      } else {
        int pos[kDmaPerWave + 1];
        chunk_pos(c, pos);
#pragma unroll
        for (int i = 0; i <= kDmaPerWave; ++i)
          __builtin_amdgcn_global_load_lds((const void*)(idx_h + pos[i]),
                                           (__attribute__((address_space(3))) void*)&kid[wave][i][0], 4, 0, 0);
      }
    };
    auto keys_landed = [&](int* key) {
      if constexpr (MODE != 2) {
#pragma unroll
        for (int i = 0; i <= kDmaPerWave; ++i) key[i] = kid[wave][i][l];
      }
    };
    // chunk c's K, V rows and biases into buffer c & 1; K and V row `row`
    // hold piece p ^ (row % kPieces) at position p, so that lanes reading one
    // piece of 16 different rows hit different banks
    auto chunk_load = [&](const int* key, uint16_t* kt, uint16_t* vt, float* bt, int32_t* kd) {
#pragma unroll
      for (int i = 0; i < kDmaPerWave; ++i) {
        const int row0 = (wave * kDmaPerWave + i) * kDmaRows;
        const int row = row0 + l / kPieces;
        const int pc = l % kPieces;
        __builtin_amdgcn_global_load_lds(
            (const void*)(kh + (uint32_t)((uint32_t)key[i] * kst_b + (uint32_t)((pc ^ (row % kPieces)) * 16))),
            (__attribute__((address_space(3))) void*)(kt + row0 * D), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void*)(vh + (uint32_t)((uint32_t)key[i] * vst_b + (uint32_t)((pc ^ (row % kPieces)) * 16))),
            (__attribute__((address_space(3))) void*)(vt + row0 * D), 16, 0, 0);
      }
      if (bh && l < 8)
        __builtin_amdgcn_global_load_lds((const void*)(bh + key[kDmaPerWave]),
                                         (__attribute__((address_space(3))) void*)(bt + 8 * wave), 4, 0, 0);
      if (MODE == 3 && l < 8) {
        for (int tb = 0; tb + 1 < ntab; ++tb)
          __builtin_amdgcn_global_load_lds(
              (const void*)(k_bucket + ((int64_t)tb * H + h) * Nk + key[kDmaPerWave]),
              (__attribute__((address_space(3))) void*)(kd + 32 * tb + 8 * wave), 4, 0, 0);
      }
    };
    const int nch = (total + 31) / 32;
    int key[kDmaPerWave + 1], key1[kDmaPerWave + 1];
    // chunk c, computed from the tiles kt, vt, bt while chunk c + 1 loads
    // into the other buffers (kn, vn, bn)
    auto chunk = [&](int c, const uint16_t* kt, const uint16_t* vt, const float* bt, const int32_t* kd,
                     uint16_t* kn, uint16_t* vn, float* bn, int32_t* kdn) {
      if (c == 0) {
        // chunk 0's rows have landed (chunk 1's, requested right behind them
        // while both buffers were free, and chunk 2's keys may still be in
        // flight: at least 2 kDmaPerWave requests were issued after them)
        static_assert(2 * kDmaPerWave < 16, "vmcnt immediate");
        if (nch > 1) __builtin_amdgcn_s_waitcnt(kWaitVm0 | (2 * kDmaPerWave));
        else __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
      } else {
        // chunk c's rows (this wave's loads) and chunk c + 1's keys have
        // landed; after the barrier every wave's loads of chunk c have, and
        // every wave is done with chunk c - 1, whose buffers chunk c + 1 takes
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        __syncthreads();
        if (c + 1 < nch) {
          keys_landed(key);
          chunk_load(key, kn, vn, bn, kdn);
        }
        if (c + 2 < nch) chunk_keys_async(c + 2, key);
      }
      const uint32_t kc = (uint32_t)(32 * c);
      // skip a chunk none of the wave's rows uses
      if (!ballot64(meets(kc, 32u))) return;
      // list and dense mode (every row's range is the whole list): a chunk
      // with all its slots inside every row's range needs no per-score masks
      // (in bucket mode the test costs more than it saves)
      bool whole = false;
      if (kList) whole = ballot64(!(kc - rlo0 < rn0 && kc + 31u - rlo0 < rn0)) == 0ull;
      float s[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        // list and dense mode: a half of the chunk none of the wave's rows
        // uses gets no scores (in bucket mode the test costs more than the
        // MFMAs it saves; the masks below leave such a half at -inf)
        const uint32_t ka = kc + (uint32_t)(16 * hf);
        if (kList && !ballot64(meets(ka, 16u))) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * hf + i] = -INFINITY;
          continue;
        }
        // A operand: chunk row 16 hf + col, dims 32c + 8g .. +8 (piece 4c + g)
        const int row = 16 * hf + col;
        bf16x8_t kop[NC];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          kop[cc] = *reinterpret_cast<const bf16x8_t*>(&kt[row * D + (((4 * cc + g) ^ (row % kPieces)) * 8)]);
        const float4 b4 = bh ? *reinterpret_cast<const float4*>(&bt[16 * hf + 4 * g])
                             : make_float4(0.f, 0.f, 0.f, 0.f);
        const float bias[4] = {b4.x * kLog2e, b4.y * kLog2e, b4.z * kLog2e, b4.w * kLog2e};
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[cc], qop[cc], sacc, 0, 0, 0);
        // sacc[i] = score(list slot 32c + 16 hf + 4 g + i, row col)
        if (whole) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s[4 * hf + i] = sacc[i] * scale_log2 + bias[i];
        } else if (MODE == 3) {
          // the slot's table is its range's; it counts unless an earlier
          // table already retains the key for this row
          int kb[3][4];
#pragma unroll
          for (int tb = 0; tb < 3; ++tb) {
            const int4 w4 = tb + 1 < ntab ? *reinterpret_cast<const int4*>(&kd[32 * tb + 16 * hf + 4 * g])
                                          : make_int4(-1, -1, -1, -1);
            kb[tb][0] = w4.x;
            kb[tb][1] = w4.y;
            kb[tb][2] = w4.z;
            kb[tb][3] = w4.w;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t j = kc + (uint32_t)(16 * hf + 4 * g + i);
            int tm = INT_MAX;
#pragma unroll
            for (int e = 0; e < E; ++e)
              if (j - rloe[e] < rne[e]) tm = min(tm, te[e]);
            bool keep = tm != INT_MAX;
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const int tb = te[e];
              if (tb < tm && tb < 3) keep = keep && kb[tb][i] != rq[e];
            }
            cnt += keep ? 1 : 0;
            s[4 * hf + i] = keep ? sacc[i] * scale_log2 + bias[i] : -INFINITY;
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t j = kc + (uint32_t)(16 * hf + 4 * g + i);
            bool in = j - rlo0 < rn0;
            if (P == 2) in = in || j - rlo1 < rn1;
            s[4 * hf + i] = in ? sacc[i] * scale_log2 + bias[i] : -INFINITY;
          }
        }
      }
      float mx = fmaxf(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])), fmaxf(fmaxf(s[4], s[5]), fmaxf(s[6], s[7])));
      mx = max_xor32(max_xor16(mx));
      const float mnew = fmaxf(m, mx);
      const float base = (mnew == -INFINITY) ? 0.f : mnew;
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(s[2 * i] - base), __builtin_amdgcn_exp2f(s[2 * i + 1] - base));
      // the sum of the rounded weights that the PV product uses
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                                __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
      // rescale the running sums only where a row's (finite) max went up
      if (ballot64(m != -INFINITY && mnew > m)) {
        const float alpha = __builtin_amdgcn_exp2f(m - base);
        lsum *= alpha;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          acc[bb][0] *= alpha;
          acc[bb][1] *= alpha;
          acc[bb][2] *= alpha;
          acc[bb][3] *= alpha;
        }
      }
      lsum += psum;
      m = mnew;
      const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      // V^T operand of block bb: lane (dim 16 bb + col, group g), slot si <->
      // chunk row 16 (si >> 2) + 4g + (si & 3), by two transposing LDS reads
      // (slots 0..3, then 4..7).  Such a read hands lane 16g + a element
      // a % 4 of the 8 bytes that lane 16g + 4e + a / 4 addresses, as its
      // element e; so this lane addresses row 4 (l >> 4) + ((l >> 2) & 3)
      // (plus 16, which has the same swizzle), dims 16 bb + 4 (l & 3) .. + 3.
      static_assert(16 % kPieces == 0, "rows r and r + 16 share their piece swizzle");
#pragma unroll
      for (int bb = 0; bb < NB; ++bb) {
        const int piece = 2 * bb + ((l & 3) >> 1);
        const uint16_t* src = vt + vrow * D + ((piece ^ (vrow % kPieces)) * 8) + (l & 1) * 4;
        const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)src);
        const v4i16_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(src + 16 * D));
        const uint2 wl = __builtin_bit_cast(uint2, lo), wh = __builtin_bit_cast(uint2, hi);
        const uint4 w = make_uint4(wl.x, wl.y, wh.x, wh.y);
        acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w), pop, acc[bb], 0, 0, 0);
      }
    };
    if (nch > 0) {
      // chunks 0 and 1 into the two (free) buffers back to back, then chunk
      // 2's keys; chunk 1's keys are requested before chunk 0's rows so that
      // waiting for them does not wait for those rows
      chunk_keys(0, key);
      if (nch > 1) chunk_keys(1, key1);
      chunk_load(key, ktA, vtA, btA, kdA);
      if (nch > 1) {
        chunk_load(key1, ktB, vtB, btB, kdB);
        if (nch > 2) chunk_keys_async(2, key);
      }
    }
    for (int c = 0; c < nch; c += 2) {
      chunk(c, ktA, vtA, btA, kdA, ktB, vtB, btB, kdB);
      if (c + 1 < nch) chunk(c + 1, ktB, vtB, btB, kdB, ktA, vtA, btA, kdA);
    }
    if (kList || (MODE == 0 && P == 1) || npass < FASTAR_WAVE) break;
    // the next batch refills both buffers: every wave is done with them
    __syncthreads();
  }
  lsum = sum_xor32(sum_xor16(lsum));
  if (MODE == 3 && n_att) {
    cnt += __shfl_xor(cnt, 16, FASTAR_WAVE);
    cnt += __shfl_xor(cnt, 32, FASTAR_WAVE);
    if (rvalid && g == 0) n_att[(int64_t)h * Nq + t] = cnt;
  }
  if (!rvalid) return;
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  // acc[b][i] = O[row col][16 b + 4 g + i].  Lanes g and g ^ 1 (l ^ 16, the
  // same row) trade halves of each block pair, so that each stores 16
  // contiguous bytes: even g dims 16 b0 + 4g .. + 7, odd g dims 16 b1 +
  // 4 (g - 1) .. + 7
  uint16_t* orow = out + ((int64_t)h * Nq + t) * D;
  const bool odd = (g & 1) != 0;
#pragma unroll
  for (int m = 0; m < NB / 2; ++m) {
    const uint2 w0 = make_uint2(pack_bf16x2(acc[2 * m][0] * inv, acc[2 * m][1] * inv),
                                pack_bf16x2(acc[2 * m][2] * inv, acc[2 * m][3] * inv));
    const uint2 w1 = make_uint2(pack_bf16x2(acc[2 * m + 1][0] * inv, acc[2 * m + 1][1] * inv),
                                pack_bf16x2(acc[2 * m + 1][2] * inv, acc[2 * m + 1][3] * inv));
    const uint2 snd = odd ? w0 : w1;
    const uint2 rcv = make_uint2(xor16_word(snd.x), xor16_word(snd.y));
    const uint4 o = odd ? make_uint4(rcv.x, rcv.y, w1.x, w1.y) : make_uint4(w0.x, w0.y, rcv.x, rcv.y);
    *reinterpret_cast<uint4*>(orow + (odd ? 16 * (2 * m + 1) + 4 * (g - 1) : 32 * m + 4 * g)) = o;
  }
  if (lse && g == 0) lse[(int64_t)h * Nq + t] = lsum > 0.f ? (m + log2f(lsum)) * kLn2 : -INFINITY;
}

// Dense attention in bf16 (every query of a head against the head's first n
// keys: all of them, or n_key_list[h]): one workgroup of 4 waves owns 128
// query rows, each wave two 16-row MFMA groups that share every LDS read of a
// chunk's K and V^T operands (half the LDS reads per score of the kernel
// above, whose one group per wave left the dense case bound by LDS
// bandwidth).  Chunks of 32 keys, their rows and biases staged in LDS as
// above (double-buffered 16-byte direct loads, swizzled rows).
template <int D>
__global__ __launch_bounds__(256, 2) void attn_dense_bf16_kernel(
    const uint16_t* __restrict__ q, int64_t q_sh, int64_t q_st, int64_t Nq,
    const uint16_t* __restrict__ k, int64_t k_sh, int64_t k_st,
    const uint16_t* __restrict__ v, int64_t v_sh, int64_t v_st, int64_t Nk,
    const float* __restrict__ key_bias, const int32_t* __restrict__ n_key_list, float scale_log2,
    uint16_t* __restrict__ out, float* __restrict__ lse, int H) {
  constexpr int RG = 2;                           // 16-row MFMA groups per wave
  constexpr int NC = D / 32;                      // k-chunks of the QK^T contraction
  constexpr int NB = D / 16;                      // 16-dim output blocks
  constexpr int kPieces = D / 8;                  // 16-byte pieces of a row
  constexpr int kDmaRows = 64 / kPieces;          // rows one 64-lane 16-byte LDS load fills
  constexpr int kDmaPerWave = 32 / kDmaRows / 4;  // such loads per wave, tile and chunk
  __shared__ __attribute__((aligned(16))) uint16_t ktA[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t ktB[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vtA[32 * D];
  __shared__ __attribute__((aligned(16))) uint16_t vtB[32 * D];
  __shared__ __attribute__((aligned(16))) float btA[32];
  __shared__ __attribute__((aligned(16))) float btB[32];
  const int64_t nbx = (Nq + 127) / 128;
  const int64_t lb = xcd_block(blockIdx.x, nbx * H);
  if (lb >= nbx * H) return;  // the whole workgroup
  const int h = (int)(lb / nbx);
  const int64_t R0 = (lb - (int64_t)h * nbx) * 128;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int l = lane_id();
  const int col = l & 15;
  const int g = l >> 4;
  const int vrow = 4 * g + ((l >> 2) & 3);
  // group gi's MFMA row of this lane: workgroup row 32 wave + 16 gi + col
  int64_t r[RG];
  bool rvalid[RG];
  bf16x8_t qop[RG][NC];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    r[gi] = R0 + 32 * wave + 16 * gi + col;
    rvalid[gi] = r[gi] < Nq;
    const uint16_t* qrow = q + (int64_t)h * q_sh + (rvalid[gi] ? r[gi] : 0) * q_st;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      uint4 u = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      if (!rvalid[gi]) u = make_uint4(0u, 0u, 0u, 0u);
      qop[gi][c] = __builtin_bit_cast(bf16x8_t, u);
    }
  }
  float m[RG], lsum[RG];
  f32x4_t acc[RG][NB];
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    m[gi] = -INFINITY;
    lsum[gi] = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[gi][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const char* kh = reinterpret_cast<const char*>(k + (int64_t)h * k_sh);
  const char* vh = reinterpret_cast<const char*>(v + (int64_t)h * v_sh);
  const uint32_t kst_b = (uint32_t)(k_st * 2), vst_b = (uint32_t)(v_st * 2);
  const float* bh = key_bias ? key_bias + (int64_t)h * Nk : nullptr;
  int total = (int)Nk;
  if (n_key_list) {
    const int64_t nl = n_key_list[h];
    total = (int)(nl < 0 ? 0 : (nl < Nk ? nl : Nk));
  }
  const int nch = (total + 31) / 32;
  // chunk c's K, V rows and biases (the keys are the positions; past the end
  // the last key, loaded and masked)
  auto chunk_load = [&](int c, uint16_t* kt, uint16_t* vt, float* bt) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i) {
      const int row0 = (wave * kDmaPerWave + i) * kDmaRows;
      const int row = row0 + l / kPieces;
      const int pc = l % kPieces;
      const uint32_t key = (uint32_t)min(32 * c + row, total - 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)(kh + (uint32_t)(key * kst_b + (uint32_t)((pc ^ (row % kPieces)) * 16))),
          (__attribute__((address_space(3))) void*)(kt + row0 * D), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const void*)(vh + (uint32_t)(key * vst_b + (uint32_t)((pc ^ (row % kPieces)) * 16))),
          (__attribute__((address_space(3))) void*)(vt + row0 * D), 16, 0, 0);
    }
    if (bh && l < 8)
      __builtin_amdgcn_global_load_lds((const void*)(bh + min(32 * c + 8 * wave + l, total - 1)),
                                       (__attribute__((address_space(3))) void*)(bt + 8 * wave), 4, 0, 0);
  };
  auto compute = [&](int c, const uint16_t* kt, const uint16_t* vt, const float* bt) {
    const int kc = 32 * c;
    const bool whole = kc + 32 <= total;  // no slot past the end
    float s[RG][8];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // A operand: chunk row 16 hf + col, dims 32 cc + 8 g .. +8 (piece 4 cc + g)
      const int row = 16 * hf + col;
      bf16x8_t kop[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        kop[cc] = *reinterpret_cast<const bf16x8_t*>(&kt[row * D + (((4 * cc + g) ^ (row % kPieces)) * 8)]);
      const float4 b4 = bh ? *reinterpret_cast<const float4*>(&bt[16 * hf + 4 * g])
                           : make_float4(0.f, 0.f, 0.f, 0.f);
      const float bias[4] = {b4.x * kLog2e, b4.y * kLog2e, b4.z * kLog2e, b4.w * kLog2e};
#pragma unroll
      for (int gi = 0; gi < RG; ++gi) {
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[cc], qop[gi][cc], sacc, 0, 0, 0);
        // sacc[i] = score(chunk slot 16 hf + 4 g + i, row col)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float sv = sacc[i] * scale_log2 + bias[i];
          s[gi][4 * hf + i] = (whole || kc + 16 * hf + 4 * g + i < total) ? sv : -INFINITY;
        }
      }
    }
    bf16x8_t pop[RG];
#pragma unroll
    for (int gi = 0; gi < RG; ++gi) {
      float mx = fmaxf(fmaxf(fmaxf(s[gi][0], s[gi][1]), fmaxf(s[gi][2], s[gi][3])),
                       fmaxf(fmaxf(s[gi][4], s[gi][5]), fmaxf(s[gi][6], s[gi][7])));
      mx = max_xor32(max_xor16(mx));
      const float mnew = fmaxf(m[gi], mx);
      const float base = (mnew == -INFINITY) ? 0.f : mnew;
      uint32_t pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[i] = pack_bf16x2(__builtin_amdgcn_exp2f(s[gi][2 * i] - base),
                            __builtin_amdgcn_exp2f(s[gi][2 * i + 1] - base));
      // the sum of the rounded weights that the PV product uses
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw[i]),
                                                __builtin_bit_cast(bf16x2_t, 0x3F803F80u), psum, false);
      // rescale the running sums only where a row's (finite) max went up
      if (ballot64(m[gi] != -INFINITY && mnew > m[gi])) {
        const float alpha = __builtin_amdgcn_exp2f(m[gi] - base);
        lsum[gi] *= alpha;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
          acc[gi][bb][0] *= alpha;
          acc[gi][bb][1] *= alpha;
          acc[gi][bb][2] *= alpha;
          acc[gi][bb][3] *= alpha;
        }
      }
      lsum[gi] += psum;
      m[gi] = mnew;
      pop[gi] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }
    // V^T operand of block bb, as in the kernel above, shared by both groups
    static_assert(16 % kPieces == 0 || kPieces == 16, "rows r and r + 16 share their piece swizzle");
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int piece = 2 * bb + ((l & 3) >> 1);
      const uint16_t* src = vt + vrow * D + ((piece ^ (vrow % kPieces)) * 8) + (l & 1) * 4;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)src);
      const v4i16_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(src + 16 * D));
      const uint2 wl = __builtin_bit_cast(uint2, lo), wh = __builtin_bit_cast(uint2, hi);
      const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, make_uint4(wl.x, wl.y, wh.x, wh.y));
#pragma unroll
      for (int gi = 0; gi < RG; ++gi)
        acc[gi][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop[gi], acc[gi][bb], 0, 0, 0);
    }
  };
  auto chunk = [&](int c, const uint16_t* kt, const uint16_t* vt, const float* bt, uint16_t* kn, uint16_t* vn,
                   float* bn) {
    if (c == 0) {
      // chunk 0's rows have landed (chunk 1's, requested right behind them,
      // may still be in flight: at least 2 kDmaPerWave requests)
      static_assert(2 * kDmaPerWave < 16, "vmcnt immediate");
      if (nch > 1) __builtin_amdgcn_s_waitcnt(kWaitVm0 | (2 * kDmaPerWave));
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    } else {
      // chunk c's rows have landed; after the barrier every wave's have, and
      // every wave is done with chunk c - 1, whose buffers chunk c + 1 takes
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      __syncthreads();
      if (c + 1 < nch) chunk_load(c + 1, kn, vn, bn);
    }
    compute(c, kt, vt, bt);
  };
  if (nch > 0) {
    chunk_load(0, ktA, vtA, btA);
    if (nch > 1) chunk_load(1, ktB, vtB, btB);
  }
  for (int c = 0; c < nch; c += 2) {
    chunk(c, ktA, vtA, btA, ktB, vtB, btB);
    if (c + 1 < nch) chunk(c + 1, ktB, vtB, btB, ktA, vtA, btA);
  }
  const bool odd = (g & 1) != 0;
#pragma unroll
  for (int gi = 0; gi < RG; ++gi) {
    const float ls = sum_xor32(sum_xor16(lsum[gi]));
    if (!rvalid[gi]) continue;
    const float inv = ls > 0.f ? 1.f / ls : 0.f;
    // as in the kernel above: lanes g and g ^ 1 trade halves of each block
    // pair so that each stores 16 contiguous bytes
    uint16_t* orow = out + ((int64_t)h * Nq + r[gi]) * D;
#pragma unroll
    for (int mb = 0; mb < NB / 2; ++mb) {
      const uint2 w0 = make_uint2(pack_bf16x2(acc[gi][2 * mb][0] * inv, acc[gi][2 * mb][1] * inv),
                                  pack_bf16x2(acc[gi][2 * mb][2] * inv, acc[gi][2 * mb][3] * inv));
      const uint2 w1 = make_uint2(pack_bf16x2(acc[gi][2 * mb + 1][0] * inv, acc[gi][2 * mb + 1][1] * inv),
                                  pack_bf16x2(acc[gi][2 * mb + 1][2] * inv, acc[gi][2 * mb + 1][3] * inv));
      const uint2 snd = odd ? w0 : w1;
      const uint2 rcv = make_uint2(xor16_word(snd.x), xor16_word(snd.y));
      const uint4 o = odd ? make_uint4(rcv.x, rcv.y, w1.x, w1.y) : make_uint4(w0.x, w0.y, rcv.x, rcv.y);
      *reinterpret_cast<uint4*>(orow + (odd ? 16 * (2 * mb + 1) + 4 * (g - 1) : 32 * mb + 4 * g)) = o;
    }
    if (lse && g == 0) lse[(int64_t)h * Nq + r[gi]] = ls > 0.f ? (m[gi] + log2f(ls)) * kLn2 : -INFINITY;
  }
}

// fp32: one query row per lane on the vector ALUs (no fp32 MFMA rounding
// concerns; the fp32 workloads are small).
template <int D, int P, int MODE>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, int64_t q_sh, int64_t q_st, int64_t Nq,
    const int32_t* __restrict__ q_bucket, const int32_t* __restrict__ q_perm,
    const float* __restrict__ k, int64_t k_sh, int64_t k_st, const float* __restrict__ v,
    int64_t v_sh, int64_t v_st, int64_t Nk, const float* __restrict__ key_bias,
    const int32_t* __restrict__ k_offsets, const int32_t* __restrict__ k_perm, int nbits,
    const int32_t* __restrict__ key_list, const int32_t* __restrict__ n_key_list, float scale,
    float* __restrict__ out, float* __restrict__ lse, int H, const int32_t* __restrict__ k_bucket, int ntab,
    int ppt, int32_t* __restrict__ n_att) {
  const int h = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= Nq) return;
  const int64_t t = (MODE == 0 || MODE == 3) ? (int64_t)q_perm[(int64_t)h * Nq + r] : r;
  float qr[D], acc[D];
  const float* qrow = q + (int64_t)h * q_sh + t * q_st;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = qrow[d];
    acc[d] = 0.f;
  }
  float m = -INFINITY, lsum = 0.f;
  const float* kh = k + (int64_t)h * k_sh;
  const float* vh = v + (int64_t)h * v_sh;
  const float* bh = key_bias ? key_bias + (int64_t)h * Nk : nullptr;
  auto attend = [&](int64_t key) {
    const float* krow = kh + key * k_st;
    float s = 0.f;
#pragma unroll
    for (int d = 0; d < D; ++d) s = fmaf(qr[d], krow[d], s);
    s = s * scale + (bh ? bh[key] : 0.f);
    const float mnew = fmaxf(m, s);
    const float alpha = expf(m - mnew);
    const float p = expf(s - mnew);
    m = mnew;
    lsum = lsum * alpha + p;
    const float* vrow = vh + key * v_st;
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = fmaf(p, vrow[d], acc[d] * alpha);
  };
  int buckets[2] = {0, -1};
  int nseg = 1;
  if (MODE == 3) {
    // the row's (table, bucket) entries, each distinct one walked once; a key
    // counts in the first table that retains it
    nseg = 0;
    int cnt = 0;
    auto probe = [&](int e) {
      const int tb = e / ppt;
      return q_bucket[(((int64_t)tb * H + h) * Nq + t) * ppt + (e - tb * ppt)];
    };
    const int ne = ntab * ppt;
    for (int e = 0; e < ne; ++e) {
      const int tb = e / ppt, b = probe(e);
      bool dup = false;
      for (int e2 = tb * ppt; e2 < e; ++e2) dup = dup || probe(e2) == b;
      if (dup) continue;
      const int64_t hb = (int64_t)tb * H + h;
      const int32_t* off = k_offsets + hb * ((1 << nbits) + 1) + (b & ((1 << nbits) - 1));
      const int32_t* idx = k_perm + hb * Nk;
      for (int64_t kk = off[0]; kk < off[1]; ++kk) {
        const int64_t key = idx[kk];
        bool earlier = false;
        for (int e2 = 0; e2 < tb * ppt; ++e2)
          earlier = earlier || k_bucket[((int64_t)(e2 / ppt) * H + h) * Nk + key] == probe(e2);
        if (earlier) continue;
        attend(key);
        ++cnt;
      }
    }
    if (n_att) n_att[(int64_t)h * Nq + t] = cnt;
  }
  if (MODE == 0) {
    const int32_t* qb = q_bucket + ((int64_t)h * Nq + t) * P;
    buckets[0] = qb[0];
    // two equal probes name one key set, walked once
    if (P == 2 && qb[1] != qb[0]) {
      buckets[1] = qb[1];
      nseg = 2;
    }
  }
  for (int sgi = 0; sgi < nseg; ++sgi) {
    int64_t kbeg = 0, kend = Nk;
    const int32_t* idx = nullptr;
    if (MODE == 0) {
      const int32_t* off = k_offsets + (int64_t)h * ((1 << nbits) + 1) + buckets[sgi];
      kbeg = off[0];
      kend = off[1];
      idx = k_perm + (int64_t)h * Nk;
    } else if (n_key_list) {  // list mode, or dense over a head's first n keys
      const int64_t nl = n_key_list[h];
      kend = nl < 0 ? 0 : (nl < Nk ? nl : Nk);
      if (MODE == 1) idx = key_list + (int64_t)h * Nk;
    }
    for (int64_t kk = kbeg; kk < kend; ++kk) attend(idx ? idx[kk] : kk);
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  float* orow = out + ((int64_t)h * Nq + t) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  if (lse) lse[(int64_t)h * Nq + t] = lsum > 0.f ? m + logf(lsum) : -INFINITY;
}

template <int D, int P, int MODE>
hipError_t launch3(const AttnArgs& a, hipStream_t s) {
  if (MODE == 2 && a.dtype == FASTAR_BF16) {
    const int64_t nb = (a.nq + 127) / 128 * a.heads;
    dim3 grid((unsigned)(FASTAR_XCDS * xcd_span(nb)));
    hipLaunchKernelGGL((attn_dense_bf16_kernel<D>), grid, dim3(256), 0, s, (const uint16_t*)a.q, a.q_sh, a.q_st,
                       a.nq, (const uint16_t*)a.k, a.k_sh, a.k_st, (const uint16_t*)a.v, a.v_sh, a.v_st, a.nk,
                       a.key_bias, a.n_key_list, a.scale * kLog2e, (uint16_t*)a.out, a.lse, a.heads);
    return hipGetLastError();
  }
  if (a.dtype == FASTAR_BF16) {
    const int64_t nb = (a.nq + 63) / 64 * a.heads;
    dim3 grid((unsigned)(FASTAR_XCDS * xcd_span(nb)));
    hipLaunchKernelGGL((attn_bf16_kernel<D, P, MODE>), grid, dim3(256), 0, s,
                       (const uint16_t*)a.q, a.q_sh, a.q_st, a.nq, a.q_bucket, a.q_perm,
                       (const uint16_t*)a.k, a.k_sh, a.k_st, (const uint16_t*)a.v, a.v_sh, a.v_st,
                       a.nk, a.key_bias, a.k_offsets, a.k_perm, a.n_bits, a.key_list,
                       a.n_key_list, a.scale * kLog2e, (uint16_t*)a.out, a.lse, a.heads, a.k_bucket,
                       a.n_tables, a.n_probes, a.n_attended);
  } else {
    dim3 grid((unsigned)((a.nq + 63) / 64), (unsigned)a.heads);
    hipLaunchKernelGGL((attn_f32_kernel<D, P, MODE>), grid, dim3(64), 0, s,
                       (const float*)a.q, a.q_sh, a.q_st, a.nq, a.q_bucket, a.q_perm,
                       (const float*)a.k, a.k_sh, a.k_st, (const float*)a.v, a.v_sh, a.v_st,
                       a.nk, a.key_bias, a.k_offsets, a.k_perm, a.n_bits, a.key_list,
                       a.n_key_list, a.scale, (float*)a.out, a.lse, a.heads, a.k_bucket, a.n_tables,
                       a.n_probes, a.n_attended);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  if (a.mode == 3) return a.n_tables * a.n_probes <= 4 ? launch3<D, 4, 3>(a, s) : launch3<D, 8, 3>(a, s);
  if (a.mode == 0) return a.n_probes == 2 ? launch3<D, 2, 0>(a, s) : launch3<D, 1, 0>(a, s);
  if (a.mode == 1) return launch3<D, 1, 1>(a, s);
  return launch3<D, 1, 2>(a, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.heads == 0 || a.nq == 0) return hipSuccess;
  return a.dim == 64 ? launch_d<64>(a, s) : launch_d<128>(a, s);
}

}  // namespace fastar
