// Direct memory->LDS tile loads for gfx950 MFMA kernels (buffer_load_dwordx4 ... lds), shared by
// the matrix products and attention.
//
// Each 16-byte load goes straight into LDS (no staging registers, no LDS write instructions),
// so NSTAGE slabs can be in flight. Loads address memory through a buffer resource set to the
// slab's origin (scalar registers) plus a 32-bit per-lane offset computed once per tile, so a load
// costs no vector address arithmetic; a load still occupies its SIMD for a few tens of cycles
// (measured: ~5% of 16 MFMAs per 1 KB load), so each slab's loads are spread evenly through the
// MFMAs of the previous slab instead of being issued in one burst.
// K-major tiles are rows of RB bytes (k contiguous) with a measured conflict-free XOR swizzle of
// the 16-byte chunks.
// Tiles stored k-row by k-row ([k][r], r contiguous) are copied as they are, with 16-byte chunk c
// of k-row k placed at chunk c ^ 4(k mod 4); their MFMA fragments are read with
// ds_read_b64_tr_b16, which hands each lane four consecutive k of one row: within a group of 16
// lanes, lane i receives element i%4 of the 8-byte rows addressed by lanes i/4, 4+i/4, 8+i/4 and
// 12+i/4, so lane j addressing k-row K0 + j/4 at column R0 + 4(j%4) gives lane i the values
// (R0 + i, K0 .. K0+3). Rows beyond the matrix are loaded from the last valid row (in bounds;
// their results are never stored).
#pragma once
#include <stdint.h>

#include "common.h"

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((ext_vector_type(4))) short s16x4;

// Raw buffer resource at byte address `p`: offsets up to 2^31 - 1, no format conversion.
DEV __amdgpu_buffer_rsrc_t buffer_at(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, 0x7fffffff, 0x00020000);
}
// 16 bytes per lane from the buffer at byte offset `voff` into LDS at `lds_wave_base` + 16 * lane.
DEV void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voff, 0, 0, 0);
}
DEV void wave_barrier_all() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int N>
DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  // vmcnt in bits [3:0] and [15:14]; expcnt (7) and lgkmcnt (15) left unconstrained
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
// Wait until at most `after` slabs of LW loads each are still in flight (after <= A).
template <int LW, int A>
DEV void wait_slabs(int after) {
  if constexpr (A == 0) {
    wait_vmcnt<0>();
  } else {
    if (after >= A) wait_vmcnt<A * LW>();
    else wait_slabs<LW, A - 1>(after);
  }
}
// vmcnt(N) and lgkmcnt(0) in one wait (this wave's LDS reads have returned)
template <int N>
DEV void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
  asm volatile("" ::: "memory");
}
template <int LW, int A>
DEV void wait_slabs_lgkm0(int after) {
  if constexpr (A == 0) {
    wait_vmcnt_lgkm0<0>();
  } else {
    if (after >= A) wait_vmcnt_lgkm0<A * LW>();
    else wait_slabs_lgkm0<LW, A - 1>(after);
  }
}

// Chunk swizzle of a tile stored k-row by k-row with R columns (2R bytes, R/8 chunks per k-row).
// A 32-lane half of ds_read_b64_tr_b16 reads 4 consecutive k-rows x 4 chunks: with k-rows of 256
// bytes or more all four rows share one 256-byte bank window, so their chunks are XORed with
// 4 (k mod 4); with 128-byte k-rows rows k and k+2 share a window, so rows 2 and 3 of each four
// XOR with 4. Either way the result stays inside the k-row.
template <int R>
DEV int tr_swz(int krow) {
  // R a multiple of 128 past 128: the XOR (< 16) stays inside the k-row's 16-chunk groups
  static_assert(R == 64 || R % 128 == 0, "transposed tiles of 64 or a multiple of 128 columns");
  if constexpr (R == 64) return ((krow >> 1) & 1) << 2;
  else return (krow & 3) << 2;
}

// K-major LDS rows of RB bytes (RB = 128 or 64): chunk swizzle measured conflict-free on gfx950
template <int RB>
DEV int swz_rb(int row) {
  if constexpr (RB == 128) return (row >> 1) & 7;
  else return (row >> 2) & 3;
}
template <int RB>
DEV int lds_off_rb(int row, int chunk) { return row * RB + ((chunk ^ swz_rb<RB>(row)) << 4); }

template <int R, bool KMAJOR, int RB, int NW = 4>
struct DmaTile {
  static constexpr int KT = RB / 2;                  // k per slab
  static constexpr int PER_WAVE = R * RB / (1024 * NW);  // 1 KB wave-loads per slab per wave
  static_assert(PER_WAVE >= 1 && PER_WAVE * 1024 * NW == R * RB, "whole wave-loads per wave");
  static constexpr int DS_PER_FRAG = KMAJOR ? 1 : 2;  // LDS read instructions per fragment
  // Byte offsets, relative to the slab origin of the tile starting at row r0, of this wave's
  // loads (one per 1 KB wave-load). They depend on the tile (rows past the matrix are clamped to
  // its last row or 8-column group, in bounds; their results are never stored), not on the slab.
  DEV static void offsets(uint32_t (&off)[PER_WAVE], int64_t ld, int r0, int r_total, int wave,
                          int lane) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int q = wave * PER_WAVE + i;
      if constexpr (KMAJOR) {
        constexpr int CPR = RB / 16, RPI = 1024 / RB;  // chunks per row, rows per wave-load
        const int row = RPI * q + lane / CPR;
        const int c = (lane % CPR) ^ swz_rb<RB>(row);
        const int r = min(r0 + row, r_total - 1);
        off[i] = (uint32_t)((int64_t)(r - r0) * ld * 2 + c * 16);
      } else {
        // the slab's k-rows are laid out one after another, 64 chunks per wave-load (a wave-load
        // may end inside a k-row when 2R does not divide 1 KB)
        constexpr int CPR = R / 8;            // 16-byte chunks per k-row
        const int pos = q * 64 + lane;
        const int krow = pos / CPR;
        const int c = (pos % CPR) ^ tr_swz<R>(krow);
        int r = r0 + c * 8;
        if (r >= r_total) r = r_total - 8;  // r_total and r0 are multiples of 8: r >= r0
        off[i] = (uint32_t)((int64_t)krow * ld * 2 + (r - r0) * 2);
      }
    }
  }
  // Buffer resource at the origin of the slab (rows from r0, k from k0).
  DEV static __amdgpu_buffer_rsrc_t slab(const bf16* base, int64_t ld, int r0, int k0) {
    return buffer_at(KMAJOR ? base + (int64_t)r0 * ld + k0 : base + (int64_t)k0 * ld + r0);
  }
  // Load i of this wave's part of a slab into the stage `dst`.
  DEV static void issue(__amdgpu_buffer_rsrc_t r, const uint32_t (&off)[PER_WAVE], int i, char* dst,
                        int wave) {
    lds_dma16(r, off[i], dst + (wave * PER_WAVE + i) * 1024);
  }
  // Fragment (32 rows from rw, k = 16s .. 16s+15 of the slab) for the calling lane.
  DEV static u32x4 frag(const char* st, int rw, int s, int lane) {
    if constexpr (KMAJOR) {
      return *reinterpret_cast<const u32x4*>(st + lds_off_rb<RB>(rw + (lane & 31), 2 * s + (lane >> 5)));
    } else {
      const int g = lane >> 4, j = lane & 15;
      const int r = rw + (g & 1) * 16 + 4 * (j & 3);
      const int chunk = r >> 3, within = (r & 7) * 2;
      u32x2 out[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int krow = 16 * s + (g >> 1) * 8 + 4 * t + (j >> 2);
        const char* a = st + krow * (2 * R) + ((chunk ^ tr_swz<R>(krow)) << 4) + within;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(a));
        out[t] = __builtin_bit_cast(u32x2, v);
      }
      return u32x4{out[0][0], out[0][1], out[1][0], out[1][1]};
    }
  }
};

// Scheduling pattern for one k-step: NM MFMAs with ND LDS reads and NV buffer loads spread evenly
// between them.
template <int NM, int ND, int NV, int Q = 0>
DEV void interleave() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int d = (Q + 1) * ND / NM - Q * ND / NM;
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);  // LDS reads
    constexpr int v = (Q + 1) * NV / NM - Q * NV / NM;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);  // buffer loads
    interleave<NM, ND, NV, Q + 1>();
  }
}

}  // namespace
