// Host-side check of the fast LDS addressing in jfa_device.h: every
// (lane_base ^ x) + y form used by the kernels must equal the reference swizzled
// offset tile_off(row, col) for all lanes and compile-time offsets in use.
#include <cstdio>

#include "jfa_device.h"

using namespace jfa;

template <int D>
int check() {
  int bad = 0;
  for (int lane = 0; lane < 64; ++lane) {
    const int c32 = lane & 31, hf = lane >> 5, t = lane & 15, g1 = (lane >> 4) & 1;
    // row reads: rows r0 + lane % 32 (r0 multiple of 16 for D = 128, of 8 for D = 64)
    const uint32_t rb = row_read_base<D>(lane);
    for (int r0 = 0; r0 < 128; r0 += (D == 128 ? 16 : 8))
      for (int ks = 0; ks < D / 16; ++ks) {
        const uint32_t fast = row_read_addr(rb, ks) + r0 * 2 * D;
        const int ref = tile_off<D>(r0 + c32, 16 * ks + 8 * hf);
        if (fast != (uint32_t)ref) ++bad;
      }
    // transposing reads, lane k offset 4*hf with K % 16 in {0, 8} and 8*hf with K % 16 in {0, 4}
    for (int kind = 0; kind < 2; ++kind) {
      const int kl = kind == 0 ? 4 * hf : 8 * hf;
      const uint32_t tb = tr_read_base<D>(lane, kl);
      for (int K = 0; K < 128; K += 4) {
        const int m = K % 16;
        if (kind == 0 && m != 0 && m != 8) continue;
        if (kind == 1 && m != 0 && m != 4) continue;
        for (int dt = 0; dt < D / 32; ++dt) {
          const uint32_t fast = tr_read_addr<D>(tb, K, dt);
          const int ref = tile_off<D>(kl + K + (t >> 2), 32 * dt + 16 * g1 + 4 * (t & 3));
          if (fast != (uint32_t)ref) ++bad;
        }
      }
    }
  }
  // direct-to-LDS copies: lane offset of copy instruction u (lds_load_tile and
  // tile_load_voff) equals row * row_bytes + swz_chunk(row, slot) * 16 for row =
  // u RPI + lane / CH (lane % CH is the LDS chunk slot the lane fills)
  {
    constexpr int CH = D / 8, RPI = 64 / CH;
    for (uint32_t row_bytes : {2u * D, 4u * D, 8u * D, 64u * D})
      for (int lane = 0; lane < 64; ++lane) {
        const uint32_t r0 = lane / CH;
        const uint32_t base = r0 * row_bytes + (((uint32_t)(lane % CH) ^ (uint32_t)swz_mask<D>((int)r0)) << 4);
        for (int u = 0; u < 64; ++u) {
          const uint32_t fast = (base ^ ((uint32_t)swz_mask<D>(u * RPI) << 4)) + (uint32_t)(u * RPI) * row_bytes;
          const int row = u * RPI + lane / CH;
          const uint32_t ref = (uint32_t)row * row_bytes + (uint32_t)swz_chunk<D>(row, lane % CH) * 16u;
          if (fast != ref) ++bad;
          if (tile_load_voff<D>(u, lane, row_bytes) != ref) ++bad;
        }
      }
  }
  // store_acc_rows read-back: (loff ^ ((RPI i mod CH) << 4)) + RPI i 2D addresses
  // row RPI i + lane / CH, chunk lane % CH of the slot swizzled by (row mod CH)
  {
    constexpr int CH = D / 8, RPI = 64 / CH;
    for (int lane = 0; lane < 64; ++lane) {
      const uint32_t c = lane % CH, r0 = lane / CH;
      const uint32_t loff = r0 * (2 * D) + ((c ^ r0) << 4);
      for (int i = 0; i < 32 / RPI; ++i) {
        const uint32_t fast = (loff ^ (uint32_t)(((RPI * i) & (CH - 1)) << 4)) + (uint32_t)(RPI * i * 2 * D);
        const uint32_t row = RPI * i + r0;
        const uint32_t ref = row * (2 * D) + ((c ^ (row & (CH - 1))) << 4);
        if (fast != ref) ++bad;
      }
    }
  }
  // the swizzle is a permutation of the 16-byte chunks of every row
  for (int row = 0; row < 64; ++row) {
    unsigned seen = 0;
    for (int c = 0; c < D / 8; ++c) seen |= 1u << swz_chunk<D>(row, c);
    if (seen != (1u << (D / 8)) - 1) ++bad;
  }
  std::printf("D=%d mismatches=%d\n", D, bad);
  return bad;
}

// join_u32 must not let a low word with bit 31 set leak into the high word (the
// buffer descriptor base is rebuilt from two readfirstlane results).
int check_join() {
  int bad = 0;
  if (join_u32(0x1u, 0x80000000u) != 0x180000000ull) ++bad;
  if (join_u32(0x7f12u, 0xfffffff0u) != 0x7f12fffffff0ull) ++bad;
  if (join_u32(0u, 0x12345678u) != 0x12345678ull) ++bad;
  std::printf("join_u32 mismatches=%d\n", bad);
  return bad;
}

int main() { return (check<128>() + check<64>() + check_join()) ? 1 : 0; }
