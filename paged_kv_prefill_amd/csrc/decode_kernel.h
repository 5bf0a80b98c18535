// Device code of the narrow attention kernel: calls with at most 32 query
// vectors per KV head (decode steps, appends of a few rows), where the work
// is streaming K/V from memory and the prefill kernel's 128-vector m tile
// would leave most of its MFMA rows empty and its workgroup with one tile in
// flight.  Included by decode.hip and decode16.hip; shares the element types
// and small helpers of attn_kernel.h.
//
// What is computed is the same as there (issue "Metal: paged-KV prefill is
// 4.43x slower than contiguous KV at 32K"; PR "perf: scale prefill attention
// splits with GPU cores on Apple7/8"): causal attention of the call's rows
// over the history and themselves, GQA head h reading KV head h / G, the key
// axis cut into splits whose partials (output normalised by its own softmax
// sum, plus its log-sum-exp) are merged by the merge kernel.
//
// Workgroup = one (split, KV head) (of one sequence, in a batch), W waves
// (8, two per SIMD, where registers and LDS allow; else 4).  Each wave owns
// every W-th 32-key tile of the split and streams it on its own: K and V
// tiles land in the wave's part of NS LDS slots by direct-to-LDS loads, NS
// tiles ahead of the tile being computed (the loads of tile t + NS are issued
// as soon as tile t has been read), so a CU keeps up to W NS tiles in flight
// with no barrier in the loop.  The query vectors of the KV head stay in
// registers as the MFMA B operand: up to 32 (32 x 32 x 16 MFMAs, one per lane
// and lane + 32) or up to 16 (16 x 16 x 32 MFMAs, one per lane % 16: half the
// matrix work when a decode step has 16 or fewer).  Each wave keeps its own
// softmax reference, sum and output accumulators; at the end the waves'
// results are combined in LDS (references are integers, so the combination
// scales by exact powers of two) into one partial per workgroup.
//
// 8-bit pages (Q8) are widened in registers at operand read time: a K read
// of 16 quants becomes the A operands of two MFMA steps (quant x scale,
// rounded once to fp16), and V^T comes from ds_read_b64_tr_b16 over byte
// pairs, which hands each lane two columns of 8 rows (8 keys) of bytes,
// scaled per key.
#pragma once

#include "attn_kernel.h"

namespace ppa {
namespace {

constexpr int kDecLds = 144 * 1024;  // LDS of the K/V slots of a workgroup
constexpr int kDecReaders = 4;     // waves that combine the workgroup's partial at the end

// Exchange bits 2 and 3 (8-bit K tiles store key swap23(m) in row m; see below).
__device__ __forceinline__ constexpr int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D, bool Q8, int NQ>
struct DecGeom {
  static constexpr int TK = 32;                          // keys per tile
  static constexpr int KT = Q8 ? TK * D : TK * D * 2;    // bytes of one K (or V) tile
  static constexpr int SCB = Q8 ? 512 : 0;              // Q8: scale rows of one K (or V) tile, 2 x 256 B
  static constexpr int WS = KT + SCB;                    // one wave's part of a slot array
  // Waves per workgroup: two per SIMD where a wave needs at most 256
  // registers (16 query vectors, or head dimension up to 128) and the LDS
  // holds a slot for each, so that one wave's loads, waits and widening
  // overlap the other's MFMAs; else one per SIMD.
  static constexpr int W = (NQ == 16 || D <= 128) && 8 * 2 * WS <= kDecLds ? 8 : 4;
  static constexpr int NS_FIT = kDecLds / (W * 2 * WS);  // slots (K and V tiles of every wave) in kDecLds
  static constexpr int NS = NS_FIT < 1 ? 1 : NS_FIT > 4 ? 4 : NS_FIT;
  static constexpr int LKQ = KT / 1024;                  // 1 KB direct-to-LDS loads per K (or V) tile
  static constexpr int LK = LKQ + (Q8 ? 2 : 0);          // loads of a K (or V) group (Q8: + two of scales)
  static constexpr int LV = LK;
  static constexpr int U = D / 16;                       // 16-byte units per 8-bit row
  static constexpr int RPL = 64 / U;                     // 8-bit rows per 1 KB load
};

// s_waitcnt vmcnt(N), other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void dec_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// Every LDS read this wave has issued has returned its data (lgkmcnt(0)),
// with the scheduler kept from moving anything across.  A slot's refill goes
// out only after this: a direct-to-LDS load does not queue behind the wave's
// LDS reads, and one with no memory to read (past the context or the wave's
// last tile) writes its zeros almost at once, so it could overwrite rows a
// read still in flight has not fetched yet.
__device__ __forceinline__ void lds_reads_done() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_sched_barrier(0);
}

// Max and sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (one column of the
// 16 x 16 MFMA layouts), every lane getting the same value: the sum adds in
// the same order on all four.
__device__ __forceinline__ float max4_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float sum4_lanes(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Signed 8-bit quants to fp16 pairs (exact), one v_cvt_f16_i16 per quant with
// the byte picked and sign-extended by SDWA: (q0, q1) and (q2, q3) of x (K:
// consecutive d), or (q0, q2) and (q1, q3) (V: byte pairs (d, d + 1) of two
// keys, split into the keys' d and d + 1).
#define PPA_Q8_PAIR(B0, B1)                                                                         \
  __device__ __forceinline__ uint32_t q8_f16_##B0##B1(uint32_t x) {                                \
    uint32_t r;                                                                                    \
    asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_" #B0 "\n\t" \
        "v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #B1 \
        : "=&v"(r)                                                                                 \
        : "v"(x));                                                                                 \
    return r;                                                                                      \
  }
PPA_Q8_PAIR(0, 1)
PPA_Q8_PAIR(2, 3)
PPA_Q8_PAIR(0, 2)
PPA_Q8_PAIR(1, 3)
#undef PPA_Q8_PAIR
__device__ __forceinline__ void q8_f16_01_23(uint32_t x, uint32_t& lo, uint32_t& hi) {
  lo = q8_f16_01(x);
  hi = q8_f16_23(x);
}
__device__ __forceinline__ void q8_f16_02_13(uint32_t x, uint32_t& ev, uint32_t& od) {
  ev = q8_f16_02(x);
  od = q8_f16_13(x);
}

template <int I, int N, class F>
__device__ __forceinline__ void dec_static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    dec_static_for<I + 1, N>(f);
  }
}

// 16-byte direct-to-LDS load (as load_lds16) over a buffer of `nrec` bytes
// from `base`: a lane whose 16 bytes end past nrec reads nothing and its LDS
// bytes are written with zeros.  The tile loop uses this for rows past the
// context's end (they arrive as zeros) and for tiles past a wave's last
// (nrec 0: every lane out of range, no memory access), so every iteration
// issues the same loads and the load counter waits below are constants.
__device__ __forceinline__ void dec_load_lds16(const char* base, uint32_t voff, uint32_t nrec, void* lds) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)scalar_ptr(base), (short)0, (int)nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds), 16, (int)voff, 0, 0, 0);
}

// The same with 4 bytes per lane (lane L writes lds + 4 L).
__device__ __forceinline__ void dec_load_lds4(const char* base, uint32_t voff, uint32_t nrec, void* lds) {
  __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)scalar_ptr(base), (short)0, (int)nrec, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds), 4, (int)voff, 0, 0, 0);
}

// LDS layouts of one wave's tiles (bank-conflict-free for the reads below):
//  * 16-bit K and V: 32 rows in 1 KB blocks of 8 rows x 8 16-byte chunks,
//    block (row / 8, chunk / 8) at (chunk / 8) 4 KB + (row / 8) 1 KB, the
//    chunk swizzled by lds_g(row) as in the prefill kernel.
//  * 8-bit K: row m (D bytes) holds key swap23(m); its 16-byte unit c sits at
//    unit c ^ sK(m).  With the swap a lane's softmax weights for one PV step
//    are 8 consecutive keys (below), so the V reads and V scales are too.
//  * 8-bit V: row = key; its 32-byte unit u sits at unit u ^ fV(key).  It is
//    read with ds_read_b64_tr_b16 taking byte pairs as 16-bit elements (see
//    the PV step).
template <int D>
__device__ __forceinline__ constexpr int dec_sk(int m) {
  constexpr int U = D / 16;
  constexpr int SH = U == 16 ? 0 : U == 8 ? 1 : 2;
  return (m >> SH) & (U - 1);
}
template <int D>
__device__ __forceinline__ constexpr int dec_fv(int key) {
  return D == 256 ? 2 * (key & 3) : D == 128 ? 2 * ((key >> 1) & 1) : 0;
}

template <int D, class E, bool PAGED, bool Q8, int NQ>
__global__ __launch_bounds__((64 * DecGeom<D, Q8, NQ>::W), 1) void attn_decode_kernel(AttnArgs a) {
  static_assert(NQ == 16 || NQ == 32, "query vectors per wave");
  using Gm = DecGeom<D, Q8, NQ>;
  constexpr int W = Gm::W;
  using M = std::conditional_t<Q8, F16, E>;   // MFMA operand type
  using vec8 = typename M::vec8;
  constexpr int TK = Gm::TK, KT = Gm::KT, WS = Gm::WS, NS = Gm::NS, LK = Gm::LK, LV = Gm::LV, LKQ = Gm::LKQ;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int EB = Q8 ? 1 : 2;
  constexpr int SROW = D / 16;   // Q8: bytes of one key's scale row
  static_assert(LV + (NS - 1) * (LK + LV) < 64 && (NS - 1) * (LK + LV) + LK < 64, "vmcnt range");
  // One array per slot and K/V, so the compiler can tell a read of one slot
  // from a direct-to-LDS load into another (it waits for a load only before
  // reads of the same array).  Unused slots are 16 bytes.
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[W * WS];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[W * WS];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[NS > 1 ? W * WS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vs1[NS > 1 ? W * WS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ks2[NS > 2 ? W * WS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vs2[NS > 2 ? W * WS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ks3[NS > 3 ? W * WS : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t vs3[NS > 3 ? W * WS : 16];
  __shared__ float ml_m[W][32], ml_l[W][32];
  // Q8: V scales of the wave's current tile, [block][key]
  __shared__ __attribute__((aligned(16))) uint16_t vst[Q8 ? W * DB * 32 : 8];

  auto kslot = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return ks0;
    else if constexpr (S == 1) return ks1;
    else if constexpr (S == 2) return ks2;
    else return ks3;
  };
  auto vslot = [&](auto s) __attribute__((always_inline)) -> uint8_t* {
    constexpr int S = decltype(s)::value;
    if constexpr (S == 0) return vs0;
    else if constexpr (S == 1) return vs1;
    else if constexpr (S == 2) return vs2;
    else return vs3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int g = blockIdx.x % a.n_kv_heads;
  const int s = (blockIdx.x / a.n_kv_heads) % a.n_splits;
  // Several sequences (a batch of decode steps): the workgroup's sequence, its
  // rows, history and block table.  A workgroup of a sequence without rows or
  // past its last split exits (the merge reads no split that starts after a
  // row's last key); the exit is uniform over the workgroup, before any barrier.
  int ws_row0 = 0;
  if (a.n_seqs > 0) {
    const int seq = blockIdx.x / (a.n_kv_heads * a.n_splits);
    const int r0 = a.cu_rows[seq];
    a.rows = a.cu_rows[seq + 1] - r0;
    a.history = a.seq_history[seq];
    a.ctx = (int)a.history + a.rows;
    if (a.rows == 0 || s * a.split_tokens >= a.ctx) return;
    a.q += (int64_t)r0 * a.n_q_heads * D;
    a.out += (int64_t)r0 * a.n_q_heads * D;
    a.bt += (int64_t)seq * a.bt_stride;
    ws_row0 = r0;
  }

  // Query vector f = (row, head) pair of the head group, row-major: lane % 32
  // (32 per wave), or lane % 16 (16 per wave; gq = lane / 16 then picks the
  // lane's share of keys and dimensions in the 16 x 16 MFMA layouts).
  const int G = a.group;
  const int nqv = a.rows * G;
  const int qv = lane & (NQ - 1);
  const int gq = lane >> 4;
  const bool qv_valid = qv < nqv;
  const int row = qv_valid ? qv / G : a.rows - 1;
  const int head = g * G + (qv_valid ? qv % G : 0);
  const int lim = (int)a.history + row;   // last key the query vector sees

  const int k0 = s * a.split_tokens;
  const int kend = min(k0 + a.split_tokens, a.ctx);
  const int n_tiles = kend > k0 ? (kend - k0 + TK - 1) / TK : 0;
  const int nt = n_tiles > wave ? (n_tiles - wave + W - 1) / W : 0;  // tiles wave + W t
  // Tiles whose keys all lie at or below the first row's last key need no mask.
  const int mask_from = (int)a.history - k0;   // tile-relative first key past row 0's limit, at tile j: - 32 j

  // Q fragments (B operand of QK).  32 vectors (32 x 32 x 16 MFMA): 16-bit
  // step ks holds d = 16 ks + 8 h + 0..7; Q8 steps 2j and 2j + 1 hold
  // d = 32 j + 16 h + 0..7 and + 8..15 (the d order of one 16-quant K read).
  // 16 vectors (16 x 16 x 32 MFMA): 16-bit step s holds d = 32 s + 8 gq + 0..7;
  // Q8 steps 2j and 2j + 1 hold d = 64 j + 16 gq + 0..7 and + 8..15.
  constexpr int QS = NQ == 16 ? D / 32 : KS;   // QK steps
  vec8 qf[QS];
  {
    const uint16_t* qp = a.q + ((int64_t)row * a.n_q_heads + head) * D;
#pragma unroll
    for (int ks = 0; ks < QS; ++ks) {
      const int d0 = NQ == 16 ? (Q8 ? 64 * (ks >> 1) + 16 * gq + 8 * (ks & 1) : 32 * ks + 8 * gq)
                              : (Q8 ? 32 * (ks >> 1) + 16 * h + 8 * (ks & 1) : 16 * ks + 8 * h);
      const u32x4 raw = qv_valid ? *(const u32x4*)(qp + d0) : u32x4{0u, 0u, 0u, 0u};
      if constexpr (std::is_same_v<M, E>) {
        qf[ks] = __builtin_bit_cast(vec8, raw);
      } else {
        // bf16 q for the fp16 MFMA: exact for |q| in fp16's normal range
        const bf16x8 qb = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (_Float16)(float)qb[e];
      }
    }
  }

  // Pool pages of the split: page p0 + l in lane l of pr0, p0 + 64 + l in pr1
  // (two plain registers: an indexed array would be moved to LDS).
  const int ps_mask = (1 << a.log2_ps) - 1;
  const int p0 = PAGED ? (k0 >> a.log2_ps) : 0;
  int pr0 = 0, pr1 = 0;
  if constexpr (PAGED) {
    const int plast = kend > k0 ? ((kend - 1) >> a.log2_ps) : p0;
    pr0 = a.bt[min(p0 + lane, plast)];
    pr1 = a.bt[min(p0 + 64 + lane, plast)];
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);   // Q and pages: nothing else is in flight in the tile loop

  const int hkvd = a.n_kv_heads * D * EB;   // bytes per token (all KV heads)
  const char* kg = (const char*)a.k + g * D * EB;
  const char* vg = (const char*)a.v + g * D * EB;
  const int ctx_last = kend - 1;

  // ---- addressing -------------------------------------------------------------
  // A tile's keys come in groups of GK consecutive keys that are consecutive
  // tokens of one page (16-bit: 8, pages hold at least 8 tokens; 8-bit: 16,
  // one scale block's rows, pages of at least 16).  Per group the tile keeps
  // the pool byte offset of its first key's row (all KV heads; the 8-bit
  // scale rows, 1/16 of the quant bytes per token, sit at 1/16 of it) and the
  // bytes of its rows that lie in the context: the loads' range, so rows
  // past the context's end arrive as zeros and a tile past the wave's last
  // (range 0) reads nothing.  K, V and the scale rows share it.
  constexpr int GK = Q8 ? 16 : 8, NG = TK / GK;
  struct TileAddr {
    int64_t off[NG];
    uint32_t nb[NG];
  };
  // Pool byte offset of key `key`'s row (wave-uniform): page from the split's
  // registers (two readlanes), place in the page.
  auto page_off = [&](int key) __attribute__((always_inline)) -> int64_t {
    const int idx = (key >> a.log2_ps) - p0;
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)pr0, idx & 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)pr1, idx & 63);
    const uint32_t page = idx >= 64 ? hi : lo;
    return ((((int64_t)page) << a.log2_ps) + (key & ps_mask)) * hkvd;
  };
  auto tile_addr = [&](int t0, bool valid) __attribute__((always_inline)) -> TileAddr {
    TileAddr ta;
    const int last = ctx_last - t0;   // tile-relative last key of the context
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int n = valid ? min(max(last - GK * gi + 1, 0), GK) : 0;
      ta.nb[gi] = (uint32_t)(n * hkvd);
      if constexpr (!PAGED) {
        ta.off[gi] = (int64_t)(t0 + GK * gi) * hkvd;
      } else if (gi == 0) {
        ta.off[0] = page_off(t0);
      } else {
        // tiles start at multiples of 32 keys: a group starts a page when its
        // tile-relative first key is a multiple of the page size
        ta.off[gi] = ((GK * gi) & ps_mask) ? ta.off[gi - 1] + (int64_t)GK * hkvd : page_off(t0 + GK * gi);
      }
    }
    return ta;
  };

  // ---- loads ----------------------------------------------------------------
  const int lrow = lane >> 3;
  // 16-bit: lane L of block (rg, cg) fetches row 8 rg + L / 8, chunk
  // 8 cg + ((L % 8) ^ lds_g(row % 16)); rg's parity picks the offset set.
  const uint32_t v16_even = lrow * hkvd + (((lane & 7) ^ lds_g(lrow)) << 4);
  const uint32_t v16_odd = lrow * hkvd + (((lane & 7) ^ lds_g(8 + lrow)) << 4);
  // 8-bit: load i covers rows RPL i .. + RPL - 1 (one 16-key group); lane L:
  // row RPL i + L / U, LDS unit w = L % U.
  constexpr int U = Gm::U, RPL = Gm::RPL;
  const int qr = lane / U, qw = lane % U;
  // Issue the loads of K (is_v false) or V of the tile `ta` describes into
  // the wave's part of slot array arr.
  // Q8: after the quants, two loads of scale rows (one per 16-key group)
  // land behind them: group b at KT + 256 b, row r (LDS row 16 b + r; K row
  // 16 b + r holds key 16 b + swap23(r)) at r SROW.
  const int s_dw = lane % (SROW / 4 > 0 ? SROW / 4 : 1);               // dword of the row
  const int s_r = min(lane / (SROW / 4 > 0 ? SROW / 4 : 1), 15);       // row within the group
  const char* ksg = (const char*)a.k_scale + g * SROW;
  const char* vsg = (const char*)a.v_scale + g * SROW;
  const int srow_bytes = a.n_kv_heads * SROW;   // scale bytes per token (all KV heads): hkvd / 16
  auto issue = [&](const TileAddr& ta, bool is_v, uint8_t* arr) __attribute__((always_inline)) {
    // The wave's offset goes through an empty asm statement so that each
    // load's LDS address is formed where the load is issued: hoisted out of
    // the loop, the (slot, load) addresses would hold dozens of scalar
    // registers for the whole loop.
    int wofs = wave * WS;
    asm volatile("" : "+s"(wofs));
    uint8_t* dst = arr + wofs;
    const char* src = is_v ? vg : kg;
    if constexpr (!Q8) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const uint32_t voff = (rg & 1) ? v16_odd : v16_even;
#pragma unroll
        for (int cg = 0; cg < D / 64; ++cg)
          dec_load_lds16(src + ta.off[rg], voff + 128 * cg, ta.nb[rg], dst + (cg * 4 + rg) * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LKQ; ++i) {
        const int m = RPL * i + qr;                            // this lane's LDS row
        const int key = is_v ? m : swap23(m);                  // its key, tile-relative
        const int grp = (RPL * i) >> 4;                        // the load's 16-key group
        const int c16 = is_v ? (qw ^ (2 * dec_fv<D>(m))) : (qw ^ dec_sk<D>(m));
        dec_load_lds16(src + ta.off[grp], (uint32_t)((key - 16 * grp) * hkvd + 16 * c16), ta.nb[grp],
                       dst + i * 1024);
      }
      const char* ssrc = is_v ? vsg : ksg;
      const int kofs = is_v ? s_r : swap23(s_r);
#pragma unroll
      for (int b = 0; b < 2; ++b)
        dec_load_lds4(ssrc + (ta.off[b] >> 4), (uint32_t)(kofs * srow_bytes + 4 * s_dw), ta.nb[b] >> 4,
                      dst + KT + 256 * b);
    }
  };

  // ---- state ----------------------------------------------------------------
  // Output accumulators: 32 vectors, O^T blocks of 32 d (32 x 32); 16
  // vectors, blocks of 16 d (16 x 16).
  constexpr int NO = NQ == 16 ? D / 16 : DB;
  using OAcc = std::conditional_t<NQ == 16, f32x4, f32x16>;
  OAcc o[NO];
#pragma unroll
  for (int db = 0; db < NO; ++db) o[db] = OAcc{};
  float m_ref = kNegInf, l = 0.f;
  const float c = a.scale_log2;

  // 16-bit operand read offsets (as in the prefill kernel, 32-row tiles).
  const int kofs16 = ((lane >> 3) & 3) * 1024 + (lane & 7) * 128 + ((h ^ lds_g(lane & 15)) << 4);
  const int v_r = 4 * h + ((lane & 15) >> 2);
  const int v_cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int vofs1 = v_r * 128 + ((v_cc ^ lds_g(v_r)) << 4) + (lane & 1) * 8;
  const int vofs2 = 1024 + v_r * 128 + ((v_cc ^ lds_g(v_r + 8)) << 4) + (lane & 1) * 8;
  // 8-bit V reads (PV step): lane 4 j + c of each 16-lane group names key
  // 16 kstep + 8 h + j (+ 4) and bytes 8 c .. + 7 of the group's 32-byte
  // unit 2 p + (lane / 16) % 2, stored at unit ^ fV(key); fV depends only on
  // key % 4 = j, so per lane it is one value.
  int tr_row[2], tr_unit[D / 64 > 0 ? D / 64 : 1];
  {
    const int trj = (lane & 15) >> 2, trc = lane & 3, gi = (lane >> 4) & 1;
    const int fv = dec_fv<D>(trj);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) tr_row[ks] = (16 * ks + 8 * h + trj) * D + 8 * trc;
#pragma unroll
    for (int p = 0; p < D / 64; ++p) tr_unit[p] = 32 * ((2 * p + gi) ^ fv);
  }

  // 16 query vectors (16 x 16 x 32 MFMAs), lane (m = lane % 16, gq):
  //  * 16-bit K: key 16 kb + m, d 32 s + 8 gq + 0..7 (chunk 4 s + gq) at
  //    kofs16q ^ (s % 2) 64 + (s / 2) 4 KB + kb 2 KB;
  //  * 16-bit V^T (ds_read_b64_tr_b16): lane 4 jv + cc of group gq names key
  //    4 gq + jv (lo; hi: + 16) and d 16 db + 4 cc + 0..3, at
  //    vofs16q ^ (db % 4) 32 + (db / 4) 4 KB (+ 2 KB);
  //  * 8-bit K: the LDS row of key 16 kb + m is 16 kb + swap23(m); read j
  //    (16 quants, d 64 j + 16 gq + 0..15) at kb 16 D + (krow16q ^ 64 j);
  //  * 8-bit V: key 4 gq + jv (+ 16), bytes 8 cc of the 32-byte unit w (at
  //    w ^ fV(key)), at trrow16q + 32 (w ^ fv16q) (+ 16 D).
  const int m16 = lane & 15, jv = (lane & 15) >> 2, cc = lane & 3;
  const int kofs16q = (m16 >> 3) * 1024 + (m16 & 7) * 128 + ((gq ^ lds_g(m16)) << 4);
  const int vofs16q = (gq >> 1) * 1024 + (4 * (gq & 1) + jv) * 128 + (((cc >> 1) ^ lds_g(4 * gq + jv)) << 4) +
                      8 * (cc & 1);
  const int krow16q = swap23(m16) * D + 16 * (gq ^ dec_sk<D>(swap23(m16)));
  const int trrow16q = (4 * gq + jv) * D + 8 * cc;
  const int fv16q = dec_fv<D>(jv);

  // One tile: QK, mask, softmax, PV; loads of tile tw + NS go out as the
  // slot's K and V are read.  `first` = the wave's first tile.
  auto tile = [&](int tw, auto slot, bool first) __attribute__((always_inline)) {
    uint8_t* kt = kslot(slot) + wave * WS;
    uint8_t* vt = vslot(slot) + wave * WS;
    const int j = wave + W * tw;
    const int t0 = k0 + TK * j;
    const bool refill = tw + NS < nt;   // the slot's next tile is one of the wave's
    const int t0n = t0 + TK * W * NS;

    // K(tw) (and its scale rows) has arrived when at most V(tw) and the K/V
    // groups of the NS - 1 later slots are outstanding.
    dec_wait_vm<LV + (NS - 1) * (LK + LV)>();

    if constexpr (NQ == 16) {
    // S^T blocks kb = 0, 1 (keys 16 kb + 0..15): sc[kb][i] is key 16 kb + 4 gq + i.
    f32x4 sc[2] = {f32x4{}, f32x4{}};
    if constexpr (!Q8) {
      constexpr int QPF = 4, NR = 2 * QS;
      i16x8 kr[NR];
      auto load = [&](int i) __attribute__((always_inline)) {   // i = 2 s + kb
        const int st = i >> 1, kb = i & 1;
        kr[i] = *LDS_PTR(const i16x8, kt + (kofs16q ^ ((st & 1) << 6)) + (st >> 1) * 4096 + kb * 2048);
      };
#pragma unroll
      for (int i = 0; i < QPF && i < NR; ++i) load(i);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (i + QPF < NR) load(i + QPF);
        sc[i & 1] = M::mfma16(__builtin_bit_cast(vec8, kr[i]), qf[i >> 1], sc[i & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      // the K scale rows of the lane's two keys
      uint32_t ksr[2][SROW / 4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kr_s = kt + KT + 256 * kb + swap23(m16) * SROW;
        if constexpr (SROW == 16) {
          const u32x4 v = *LDS_PTR(const u32x4, kr_s);
#pragma unroll
          for (int e = 0; e < 4; ++e) ksr[kb][e] = v[e];
        } else if constexpr (SROW == 8) {
          const u32x2 v = *LDS_PTR(const u32x2, kr_s);
          ksr[kb][0] = v[0];
          ksr[kb][1] = v[1];
        } else {
          ksr[kb][0] = *LDS_PTR(const uint32_t, kr_s);
        }
      }
      constexpr int NR = 2 * (D / 64), QPF = NR < 3 ? NR : 3;
      const uint32_t ksel = (gq >> 1) ? 0x03020302u : 0x01000100u;
      u32x4 kr[NR];
      auto load = [&](int i) __attribute__((always_inline)) {   // i = 2 j + kb
        kr[i] = *LDS_PTR(const u32x4, kt + (i & 1) * 16 * D + (krow16q ^ (64 * (i >> 1))));
      };
#pragma unroll
      for (int i = 0; i < QPF; ++i) load(i);
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        if (i + QPF < NR) load(i + QPF);
        const int jr = i >> 1, kb = i & 1;
        // the read's scale block is 2 jr + gq / 2: half gq / 2 of dword jr, both halves
        const h2 ss = __builtin_bit_cast(h2, __builtin_amdgcn_perm(ksr[kb][jr], ksr[kb][jr], ksel));
        uint32_t w[8];
        uint32_t qh[8];   // the quants exactly in fp16 (all first: each conversion's result is read later)
#pragma unroll
        for (int k = 0; k < 4; ++k) q8_f16_01_23(kr[i][k], qh[2 * k], qh[2 * k + 1]);
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, qh[k]) * ss);   // rounded once
        const u32x4 a0 = {w[0], w[1], w[2], w[3]}, a1 = {w[4], w[5], w[6], w[7]};
        sc[kb] = M::mfma16(__builtin_bit_cast(vec8, a0), qf[2 * jr], sc[kb]);
        sc[kb] = M::mfma16(__builtin_bit_cast(vec8, a1), qf[2 * jr + 1], sc[kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // This slot's K has been read: its next tile's K group goes out.
    const TileAddr tan = tile_addr(t0n, refill);
    lds_reads_done();
    issue(tan, false, kslot(slot));

    if (TK * j + TK - 1 > mask_from) {
      const int rel = lim - t0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][i] = 16 * kb + 4 * gq + i > rel ? kNegInf : sc[kb][i];
    }
    if (first) {
      float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) mx = fmaxf(mx, fmaxf(sc[0][i], sc[1][i]));
      m_ref = ceilf(max4_lanes(mx) * c);
    }
    // P: PV K index i = keys 4 gq + i (i < 4) and 16 + 4 gq + i - 4: the lane's own scores.
    vec8 pb;
    float rs = 0.f;
    auto weights = [&]() __attribute__((always_inline)) {
      const float base = m_ref == kNegInf ? 0.f : m_ref;
      float p32[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p32[i] = __builtin_amdgcn_exp2f(fmaf(sc[i >> 2][i & 3], c, -base));
      pb = M::from_f32(p32);
      rs = M::sum8(pb, 0.f);
    };
    weights();
    if (__builtin_expect(__ballot(!(l + rs <= kSumLimit)) != 0, 0)) {
      float mx = fmaxf(sc[0][0], sc[1][0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) mx = fmaxf(mx, fmaxf(sc[0][i], sc[1][i]));
      const float m_new = fmaxf(m_ref, ceilf(max4_lanes(mx) * c));
      if (m_new != kNegInf && m_new != m_ref) {
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NO; ++db) o[db] *= alpha;
        m_ref = m_new;
      }
      weights();
    }
    l += rs;

    dec_wait_vm<(NS - 1) * (LK + LV) + LK>();
    if constexpr (Q8) {
      if (h == 0) {
        const int key = lane & 31;
        const uint8_t* vr = vt + KT + 256 * (key >> 4) + (key & 15) * SROW;
        uint32_t w4[SROW / 4];
        if constexpr (SROW == 16) {
          const u32x4 v = *LDS_PTR(const u32x4, vr);
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = v[e];
        } else if constexpr (SROW == 8) {
          const u32x2 v = *LDS_PTR(const u32x2, vr);
          w4[0] = v[0];
          w4[1] = v[1];
        } else {
          w4[0] = *LDS_PTR(const uint32_t, vr);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t w2 = w4[db >> 1];
          const uint16_t sc16 = (uint16_t)((db & 1) ? (w2 >> 16) : (w2 & 0xffffu));
          vst[(wave * DB + db) * 32 + key] = sc16;
        }
      }
    }
    if constexpr (!Q8) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int ofs = (vofs16q ^ ((db & 3) << 5)) + (db >> 2) * 4096;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + ofs));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + ofs + 2048));
        const vec8 av = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = M::mfma16(av, pb, o[db]);
      }
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int w = 0; w < D / 32; ++w) {
        const int ofs = trrow16q + 32 * (w ^ fv16q);
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + ofs)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            LDS_PTR(i16x4, vt + ofs + 16 * D)));
        // scales of keys 4 gq + 0..3 and 16 + 4 gq + 0..3 at block w
        const u32x2 svl = *LDS_PTR(const u32x2, (uint8_t*)vst + ((wave * DB + w) * 32 + 4 * gq) * 2);
        const u32x2 svh = *LDS_PTR(const u32x2, (uint8_t*)vst + ((wave * DB + w) * 32 + 16 + 4 * gq) * 2);
        const uint32_t x[4] = {lo[0], lo[1], hi[0], hi[1]};
        const uint32_t sk4[4] = {svl[0], svl[1], svh[0], svh[1]};
        uint32_t we[4], wo[4], ev[4], od[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q8_f16_02_13(x[k], ev[k], od[k]);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t sk = sk4[k];
          const h2 sc2 = __builtin_bit_cast(h2, sk);
          we[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, ev[k]) * sc2);
          wo[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, od[k]) * sc2);
        }
        o[2 * w] = M::mfma16(__builtin_bit_cast(vec8, u32x4{we[0], we[1], we[2], we[3]}), pb, o[2 * w]);
        o[2 * w + 1] = M::mfma16(__builtin_bit_cast(vec8, u32x4{wo[0], wo[1], wo[2], wo[3]}), pb, o[2 * w + 1]);
      }
    }
    lds_reads_done();
    issue(tan, true, vslot(slot));
    } else {
    f32x16 sc = f32x16{};
    if constexpr (!Q8) {
      constexpr int QPF = 4;
      i16x8 kr[KS];
      auto load = [&](int ks) __attribute__((always_inline)) {
        kr[ks] = *LDS_PTR(const i16x8, kt + (kofs16 ^ ((ks & 3) << 5)) + (ks >> 2) * 4096);
      };
#pragma unroll
      for (int ks = 0; ks < QPF && ks < KS; ++ks) load(ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + QPF < KS) load(ks + QPF);
        sc = M::mfma(__builtin_bit_cast(vec8, kr[ks]), qf[ks], sc);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      // The K scale row of this lane's LDS row (single vector loads: the
      // compiler keeps their alias information).
      uint32_t ksr[SROW / 4];
      {
        const int m = lane & 31;
        const uint8_t* kr_s = kt + KT + 256 * (m >> 4) + (m & 15) * SROW;
        if constexpr (SROW == 16) {
          const u32x4 v = *LDS_PTR(const u32x4, kr_s);
#pragma unroll
          for (int e = 0; e < 4; ++e) ksr[e] = v[e];
        } else if constexpr (SROW == 8) {
          const u32x2 v = *LDS_PTR(const u32x2, kr_s);
          ksr[0] = v[0];
          ksr[1] = v[1];
        } else {
          ksr[0] = *LDS_PTR(const uint32_t, kr_s);
        }
      }
      const int m = lane & 31;
      const uint8_t* krow = kt + m * D;
      constexpr int QPF = DB < 3 ? DB : 3;
      u32x4 kr[DB];
      auto load = [&](int jj) __attribute__((always_inline)) {
        kr[jj] = *LDS_PTR(const u32x4, krow + 16 * ((2 * jj + h) ^ dec_sk<D>(m)));
      };
#pragma unroll
      for (int jj = 0; jj < QPF; ++jj) load(jj);
#pragma unroll
      for (int jj = 0; jj < DB; ++jj) {
        if (jj + QPF < DB) load(jj + QPF);
        // scale jj: half jj % 2 of dword jj / 2, both halves
        const h2 ss = __builtin_bit_cast(h2, __builtin_amdgcn_perm(ksr[jj >> 1], ksr[jj >> 1],
                                                                   (jj & 1) ? 0x03020302u : 0x01000100u));
        uint32_t w[8];
        uint32_t qh[8];   // the quants exactly in fp16 (all first: each conversion's result is read later)
#pragma unroll
        for (int k = 0; k < 4; ++k) q8_f16_01_23(kr[jj][k], qh[2 * k], qh[2 * k + 1]);
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, qh[k]) * ss);   // rounded once
        const u32x4 a0 = {w[0], w[1], w[2], w[3]}, a1 = {w[4], w[5], w[6], w[7]};
        sc = M::mfma(__builtin_bit_cast(vec8, a0), qf[2 * jj], sc);
        sc = M::mfma(__builtin_bit_cast(vec8, a1), qf[2 * jj + 1], sc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // This slot's K has been read: its next tile's K group goes out.
    const TileAddr tan = tile_addr(t0n, refill);
    lds_reads_done();
    issue(tan, false, kslot(slot));

    // Element e of sc is S^T row 8 (e / 4) + 4 h + e % 4 (Q8: key swap23 of it).
    auto key_of = [&](int e) __attribute__((always_inline)) {
      const int r = 8 * (e >> 2) + 4 * h + (e & 3);
      return Q8 ? swap23(r) : r;
    };
    if (TK * j + TK - 1 > mask_from) {
      const int rel = lim - t0;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = key_of(e) > rel ? kNegInf : sc[e];
    }

    // Softmax weights against the integer reference (see kSumLimit): the
    // wave's first tile sets it; a tile whose sum would overflow raises it.
    if (first) {
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      m_ref = ceilf(max_with_partner(mx) * c);
    }
    vec8 pb[2];
    float rs = 0.f;
    auto weights = [&]() __attribute__((always_inline)) {
      const float base = m_ref == kNegInf ? 0.f : m_ref;
      float p32[16];
      rs = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p32[e] = __builtin_amdgcn_exp2f(fmaf(sc[e], c, -base));
        if ((e & 7) == 7) {
          pb[e >> 3] = M::from_f32(p32 + (e & ~7));
          rs = M::sum8(pb[e >> 3], rs);
        }
      }
    };
    weights();
    if (__builtin_expect(__ballot(!(l + rs <= kSumLimit)) != 0, 0)) {
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      const float m_new = fmaxf(m_ref, ceilf(max_with_partner(mx) * c));
      if (m_new != kNegInf && m_new != m_ref) {
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);   // 2^-k, 0 if m_ref was -inf
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NO; ++db) o[db] *= alpha;
        m_ref = m_new;
      }
      weights();
    }
    l += rs;

    // V(tw) has arrived when at most the later slots' groups and the K group
    // just issued are outstanding.
    dec_wait_vm<(NS - 1) * (LK + LV) + LK>();
    if constexpr (Q8) {
      // The V scale rows of this tile, transposed to [block][key] for the PV
      // reads (lanes 0-31, one key each).
      if (h == 0) {
        const int key = lane & 31;
        const uint8_t* vr = vt + KT + 256 * (key >> 4) + (key & 15) * SROW;
        uint32_t w4[SROW / 4];
        if constexpr (SROW == 16) {
          const u32x4 v = *LDS_PTR(const u32x4, vr);
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = v[e];
        } else if constexpr (SROW == 8) {
          const u32x2 v = *LDS_PTR(const u32x2, vr);
          w4[0] = v[0];
          w4[1] = v[1];
        } else {
          w4[0] = *LDS_PTR(const uint32_t, vr);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t w2 = w4[db >> 1];
          const uint16_t sc16 = (uint16_t)((db & 1) ? (w2 >> 16) : (w2 & 0xffffu));
          vst[(wave * DB + db) * 32 + key] = sc16;
        }
      }
    }

    // O^T[d][qv] += V^T[d][key] P^T[key][qv], 16 keys per MFMA.
#pragma unroll
    for (int kstep = 0; kstep < 2; ++kstep) {
      if constexpr (!Q8) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          // rows 16 kstep + 4 h + (lane % 16) / 4 and + 8 (the keys of pb[kstep])
          const int imm = (db >> 1) * 4096 + kstep * 2048;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs1 ^ ((db & 1) << 6)) + imm));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, vt + (vofs2 ^ ((db & 1) << 6)) + imm));
          const vec8 av = __builtin_bit_cast(vec8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[db] = M::mfma(av, pb[kstep], o[db]);
        }
      } else {
        // 8-bit V, 64 values of d per step p: each 16-lane group reads 4 keys
        // x 32 bytes with ds_read_b64_tr_b16 (lane 4 j + c names key row j,
        // bytes 8 c .. + 7), lo for keys 16 kstep + 8 h + 0..3 and hi for
        // + 4..7; lane L then holds the byte pair (d, d + 1), d = 64 p + 2 (L % 32),
        // of 8 keys.  Even bytes make the A operand of o[2 p] (row m: d =
        // 64 p + 2 m), odd bytes that of o[2 p + 1] (d + 1), each widened with
        // the keys' scales of block d / 32.
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const int gi = (lane >> 4) & 1;
#pragma unroll
        for (int p = 0; p < D / 64; ++p) {
          const int u = 2 * p + gi;   // 32-byte unit of the group's window
          // one offset per read from the slot base (a long chain of address
          // steps would lose the compiler's alias information)
          const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              LDS_PTR(i16x4, vt + (tr_row[kstep] + tr_unit[p]))));
          const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              LDS_PTR(i16x4, vt + (tr_row[kstep] + 4 * D + tr_unit[p]))));
          // scales of keys 16 kstep + 8 h + 0..7 at block 2 p + gi
          const u32x4 sv = *LDS_PTR(const u32x4, (uint8_t*)vst + ((wave * DB + u) * 32 + 16 * kstep + 8 * h) * 2);
          const uint32_t x[4] = {lo[0], lo[1], hi[0], hi[1]};
          // x[k] = bytes (d, d + 1) of keys 2k and 2k + 1
          uint32_t we[4], wo[4], ev[4], od[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) q8_f16_02_13(x[k], ev[k], od[k]);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            // (the element goes through a plain variable: a bit cast of a
            // vector element as such reads element 0)
            const uint32_t sk = sv[k];
            const h2 sc2 = __builtin_bit_cast(h2, sk);
            we[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, ev[k]) * sc2);
            wo[k] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, od[k]) * sc2);
          }
          o[2 * p] = M::mfma(__builtin_bit_cast(vec8, u32x4{we[0], we[1], we[2], we[3]}), pb[kstep], o[2 * p]);
          o[2 * p + 1] = M::mfma(__builtin_bit_cast(vec8, u32x4{wo[0], wo[1], wo[2], wo[3]}), pb[kstep], o[2 * p + 1]);
        }
      }
    }
    // This slot's V has been read: its next tile's V group goes out.
    lds_reads_done();
    issue(tan, true, vslot(slot));
    }
  };

  // ---- tile loop ------------------------------------------------------------
  // Prologue: the first NS tiles' K and V groups, in tile order.
  auto prologue = [&](auto slot) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    const int t0 = k0 + TK * (wave + W * SL);
    const TileAddr ta = tile_addr(t0, SL < nt);
    issue(ta, false, kslot(slot));
    issue(ta, true, vslot(slot));
  };
  prologue(std::integral_constant<int, 0>{});
  if constexpr (NS > 1) prologue(std::integral_constant<int, 1>{});
  if constexpr (NS > 2) prologue(std::integral_constant<int, 2>{});
  if constexpr (NS > 3) prologue(std::integral_constant<int, 3>{});
  // Whole groups of NS tiles, then the remainder with nested conditions: on
  // every path the slots run in order, so the compiler's own load counting
  // agrees with the waits above (a path that skips a slot and runs a later
  // one would make it wait for every load in flight).
  int t = 0;
  for (; t + NS <= nt; t += NS) {
    tile(t, std::integral_constant<int, 0>{}, t == 0);
    if constexpr (NS > 1) tile(t + 1, std::integral_constant<int, 1>{}, false);
    if constexpr (NS > 2) tile(t + 2, std::integral_constant<int, 2>{}, false);
    if constexpr (NS > 3) tile(t + 3, std::integral_constant<int, 3>{}, false);
  }
  if constexpr (NS > 1) {
    if (t < nt) {
      tile(t, std::integral_constant<int, 0>{}, t == 0);
      if constexpr (NS > 2) {
        if (t + 1 < nt) {
          tile(t + 1, std::integral_constant<int, 1>{}, false);
          if constexpr (NS > 3)
            if (t + 2 < nt) tile(t + 2, std::integral_constant<int, 2>{}, false);
        }
      }
    }
  }

  // ---- combine the waves -----------------------------------------------------
  // Each wave leaves its reference, sum and unnormalised accumulators; its own
  // slots (all loads consumed) hold the accumulators as blocks of SB bytes,
  // bj = 4 db + jq of [h][qv][4 floats], d = 32 db + 8 jq + 4 h + 0..3.
  dec_wait_vm<0>();
  const float l_tot = NQ == 16 ? sum4_lanes(l) : sum_with_partner(l);
  if (lane < NQ) {
    ml_m[wave][qv] = m_ref;
    ml_l[wave][qv] = l_tot;
  }
  constexpr int SB = 32 * NQ;     // bytes of one staging block
  constexpr int BPA = KT / SB;    // staging blocks per slot array part (a wave's part of one array)
  static_assert(2 * NS * BPA >= 4 * DB, "the output staging fits the wave's slots");
  auto arr_of = [&](auto ai) __attribute__((always_inline)) -> uint8_t* {
    constexpr int A = decltype(ai)::value;
    if constexpr (A == 0) return ks0;
    else if constexpr (A == 1) return vs0;
    else if constexpr (A == 2) return ks1;
    else if constexpr (A == 3) return vs1;
    else if constexpr (A == 4) return ks2;
    else if constexpr (A == 5) return vs2;
    else if constexpr (A == 6) return ks3;
    else return vs3;
  };
  // Array A0 + k for k < N known at run time (after the tile loop only: a
  // pointer chosen among the arrays at run time inside it would keep the
  // compiler from telling the arrays apart there).
  auto arr_rt = [&](auto a0c, auto nc, int k) __attribute__((always_inline)) -> uint8_t* {
    constexpr int A0 = decltype(a0c)::value, N = decltype(nc)::value;
    uint8_t* p = arr_of(std::integral_constant<int, A0>{});
    if constexpr (N > 1) p = k == 1 ? arr_of(std::integral_constant<int, A0 + 1>{}) : p;
    if constexpr (N > 2) p = k == 2 ? arr_of(std::integral_constant<int, A0 + 2>{}) : p;
    if constexpr (N > 3) p = k == 3 ? arr_of(std::integral_constant<int, A0 + 3>{}) : p;
    return p;
  };
  // blocks BJ0 + k (k < KN at run time, all in one array) of this wave: byte address
  auto stage = [&](auto bjc, auto knc, int k) __attribute__((always_inline)) -> uint8_t* {
    constexpr int BJ0 = decltype(bjc)::value, KN = decltype(knc)::value;
    static_assert(BJ0 / BPA == (BJ0 + KN - 1) / BPA, "the blocks lie in one array");
    return arr_of(std::integral_constant<int, BJ0 / BPA>{}) + wave * WS + (BJ0 % BPA + k) * SB;
  };
  using I1 = std::integral_constant<int, 1>;
  if constexpr (NQ == 32 && !Q8) {
    dec_static_for<0, 4 * DB>([&](auto bjc) __attribute__((always_inline)) {
      constexpr int BJ = decltype(bjc)::value;
      constexpr int DBI = BJ / 4, JQ = BJ % 4;
      const f32x4 v4 = {o[DBI][4 * JQ], o[DBI][4 * JQ + 1], o[DBI][4 * JQ + 2], o[DBI][4 * JQ + 3]};
      *(f32x4*)(stage(bjc, I1{}, 0) + (h * 32 + qv) * 16) = v4;
    });
  } else if constexpr (NQ == 32) {
    // o[2 p + par] row m = 8 j + 4 h + i holds d = 64 p + 16 j + 8 h + 2 i + par:
    // four consecutive d = 64 p + 16 j + 8 h + 4 f + 0..3 (f = i / 2) go to
    // block 4 (2 p + j / 2) + 2 (j % 2) + h, half f.
    dec_static_for<0, D / 8>([&](auto c) __attribute__((always_inline)) {   // (P, J, F): D/64 x 4 x 2
      constexpr int C = decltype(c)::value;
      constexpr int P = C / 8, J = (C / 2) % 4, F = C % 2;
      constexpr int BJ0 = 4 * (2 * P + J / 2) + 2 * (J % 2);
      const f32x4 v4 = {o[2 * P][4 * J + 2 * F], o[2 * P + 1][4 * J + 2 * F], o[2 * P][4 * J + 2 * F + 1],
                        o[2 * P + 1][4 * J + 2 * F + 1]};
      *(f32x4*)(stage(std::integral_constant<int, BJ0>{}, std::integral_constant<int, 2>{}, h) + (F * 32 + qv) * 16) = v4;
    });
  } else if constexpr (!Q8) {
    // o[db] element i holds d = 16 db + 4 gq + i: block 4 (db / 2) + 2 (db % 2) + gq / 2, h = gq % 2
    dec_static_for<0, D / 16>([&](auto dbc) __attribute__((always_inline)) {
      constexpr int DBI = decltype(dbc)::value;
      constexpr int BJ0 = 4 * (DBI / 2) + 2 * (DBI % 2);
      *(f32x4*)(stage(std::integral_constant<int, BJ0>{}, std::integral_constant<int, 2>{}, gq >> 1) +
                ((gq & 1) * 16 + qv) * 16) = o[DBI];
    });
  } else {
    // o[2 w + par] element i holds d = 32 w + 8 gq + 2 i + par: d = 32 w + 8 gq + 4 f + 0..3
    // go to block 4 w + gq, h = f
    dec_static_for<0, D / 16>([&](auto c) __attribute__((always_inline)) {   // (Wd, F)
      constexpr int C = decltype(c)::value;
      constexpr int Wd = C / 2, F = C % 2;
      const f32x4 v4 = {o[2 * Wd][2 * F], o[2 * Wd + 1][2 * F], o[2 * Wd][2 * F + 1], o[2 * Wd + 1][2 * F + 1]};
      uint8_t* dst;
      if constexpr (BPA % 4 == 0) {
        dst = stage(std::integral_constant<int, 4 * Wd>{}, std::integral_constant<int, 4>{}, gq);
      } else {
        static_assert(BPA == 2, "staging blocks per array");
        dst = (gq < 2 ? stage(std::integral_constant<int, 4 * Wd>{}, std::integral_constant<int, 2>{}, gq)
                      : stage(std::integral_constant<int, 4 * Wd + 2>{}, std::integral_constant<int, 2>{}, gq - 2));
      }
      *(f32x4*)(dst + (F * 16 + qv) * 16) = v4;
    });
  }
  __syncthreads();

  // The first kDecReaders waves over the NQ x D/4 four-float units: step i
  // takes BPS blocks bj = BPS i + t / (2 NQ), unit (h, qv) = t % (2 NQ) of the
  // block, and sums it over the W waves.
  const int wq = tid >> 6;
  if (wq >= kDecReaders) return;
  constexpr int UB = 2 * NQ, BPS = 64 * kDecReaders / UB;
  static_assert((4 * DB) % BPS == 0, "whole steps");
  const int bis = tid / UB, unit = tid % UB;
  const int uh = unit / NQ, uq = unit % NQ;
  const int64_t pairs = (int64_t)a.ws_rows * a.n_q_heads;   // workspace pairs per split
  float mw[W], lw[W], mx = kNegInf;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    mw[w] = ml_m[w][uq];
    lw[w] = ml_l[w][uq];
    mx = fmaxf(mx, mw[w]);
  }
  float sw[W], lsum = 0.f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    // a wave that saw no key of this query vector adds nothing
    sw[w] = (mw[w] == kNegInf || !(lw[w] > 0.f)) ? 0.f : __builtin_amdgcn_exp2f(mw[w] - mx);   // exact: integers
    lsum += sw[w] * lw[w];
  }
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const int urow = uq / G, uhead = g * G + uq % G;
  const int64_t pair = (int64_t)urow * a.n_q_heads + uhead;                  // in the call's (sequence's) output
  const int64_t wpair = (int64_t)(ws_row0 + urow) * a.n_q_heads + uhead;    // in the workspace
  const bool uvalid = uq < nqv;
  dec_static_for<0, 4 * DB / BPS>([&](auto ic) __attribute__((always_inline)) {
    constexpr int I = decltype(ic)::value;
    constexpr int B0 = BPS * I;   // the step's first block
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    uint8_t* base;
    if constexpr (BPA % BPS == 0) {
      base = arr_of(std::integral_constant<int, B0 / BPA>{}) + (B0 % BPA + bis) * SB;
    } else {
      static_assert(BPS % BPA == 0 && BPS / BPA <= 4, "a step's blocks over whole arrays");
      base = arr_rt(std::integral_constant<int, B0 / BPA>{}, std::integral_constant<int, BPS / BPA>{}, bis / BPA) +
             (bis % BPA) * SB;
    }
#pragma unroll
    for (int w = 0; w < W; ++w) acc += sw[w] * *(const f32x4*)(base + w * WS + (uh * NQ + uq) * 16);
    if (!uvalid) return;
    const int bj = B0 + bis;
    const int d = 32 * (bj >> 2) + 8 * (bj & 3) + 4 * uh;
    if (a.n_splits == 1) {
      const uint32_t lo = E::bits(acc[0] * inv) | ((uint32_t)E::bits(acc[1] * inv) << 16);
      const uint32_t hi = E::bits(acc[2] * inv) | ((uint32_t)E::bits(acc[3] * inv) << 16);
      *(u32x2*)(a.out + pair * D + d) = u32x2{lo, hi};
    } else {
      *(f32x4*)(a.ws_o + ((int64_t)s * pairs + wpair) * D + d) =
          f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    }
  });
  if (a.n_splits > 1 && uvalid && bis == 0 && uh == 0)
    a.ws_lse[(int64_t)s * pairs + wpair] = lsum > 0.f ? mx + log2f(lsum) : kNegInf;
}

template <int D, class E, bool PAGED, bool Q8, int NQ>
hipError_t launch_decode_t(const AttnArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_decode_kernel<D, E, PAGED, Q8, NQ>), dim3(grid), dim3(64 * DecGeom<D, Q8, NQ>::W), 0, stream, a);
  return hipGetLastError();
}

template <class E, bool PAGED, bool Q8, int NQ>
hipError_t launch_decode_d(const AttnArgs& a, int head_dim, int grid, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_decode_t<64, E, PAGED, Q8, NQ>(a, grid, stream);
    case 128: return launch_decode_t<128, E, PAGED, Q8, NQ>(a, grid, stream);
    case 256: return launch_decode_t<256, E, PAGED, Q8, NQ>(a, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

// Every instantiation for NQ query vectors per wave (32: 8-bit pages only;
// 16-bit calls of 17-32 vectors run the prefill kernel).
template <int NQ>
hipError_t launch_decode_nq(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                            hipStream_t stream) {
  auto by_e = [&](auto e) {
    using E = decltype(e);
    if (q8) return launch_decode_d<E, true, true, NQ>(a, head_dim, grid, stream);
    if constexpr (NQ == 16) {
      if (paged) return launch_decode_d<E, true, false, NQ>(a, head_dim, grid, stream);
      return launch_decode_d<E, false, false, NQ>(a, head_dim, grid, stream);
    } else {
      return hipErrorInvalidValue;
    }
  };
  return dtype == 1 ? by_e(BF16{}) : by_e(F16{});
}

}  // namespace

// 16 query vectors per wave (16 x 16 MFMAs), defined in decode16.hip.
hipError_t launch_attention_decode16(const AttnArgs& a, int head_dim, int dtype, bool paged, bool q8, int grid,
                                     hipStream_t stream);

}  // namespace ppa
