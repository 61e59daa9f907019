// Internal declarations shared by the C ABI (vkv_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <stddef.h>
#include <stdint.h>

#include "verkv.h"

namespace vkv {

// Carves 256-byte aligned regions out of one caller workspace.
struct Carve {
  size_t off = 0;
  template <typename T>
  size_t take(size_t count) {
    off = (off + 255) & ~size_t(255);
    const size_t o = off;
    off += count * sizeof(T);
    return o;
  }
};

template <typename T>
static inline T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

// ------------------------------------------------------------ compression
constexpr int kCompChunk = 4096;   // tokens per workgroup
constexpr int kCompBins = 2048;    // 11-bit radix digits over 33-bit scores

struct CompressSlice {
  uint64_t lo;        // lower edge of the current bracket of score values
  uint64_t s_below;   // sum of free scores below the bracket
  uint64_t num, den;  // water level c = num / den (grid units); den 0 => inf
  uint32_t c_above;   // free tokens at or above the bracket's upper edge
  uint32_t n_free;    // free (non-forced) tokens
  int32_t done;       // water level known
  int32_t all_sat;    // every free token saturates (L empty)
  uint32_t pad[4];
};

struct CompressLayout {
  int n_slices, ncc, nwords;
  size_t slices, hcnt, hsum, ccnt, bits, total;
};

CompressLayout compress_layout(const vkv_compress_args &a);
hipError_t launch_compress(const vkv_compress_args &a, const CompressLayout &L,
                           int64_t b_free, int32_t n_forced, hipStream_t s);
// (k and v are device-readable addresses: device memory, or pinned host
// memory's device view)

// ------------------------------------------------------------ decoding
struct DecodeLayout {
  int grp, nch, nrr, ncr, ncf, npad, nwords, chunk, nrc, nsub, rsub, nsel;
  int spec_m;  // rows per (request, KV head) read ahead (0: none)
  size_t sp_hist, sp_cnt, sp_res, sp_bits, sp_base, sp_list, spec_kv;
  size_t shat, ell, hpart, fstat, fbits, hbits, pmax, p0part, hres, rows,
      bpart, band,
      bstate,
      rbeta, binst, bhist, bcnt, bkeys, bav, cpart, ccount, clo, tpart, candk, candw, candq, dpart,
      rpart, apart, aparto, skey, total;
};

DecodeLayout decode_layout(const vkv_decode_args &a);
int decode_phase_count();
const char *decode_phase_name(int i);
hipError_t launch_decode(const vkv_decode_args &a, const DecodeLayout &L,
                         const uint16_t *host_kv_dev, hipStream_t s);

// ------------------------------------------------------------ 2-bit sketch
struct Sketch2Layout {
  int nblk;
  size_t part, total;
};

Sketch2Layout sketch2_layout(const vkv_sketch2_args &a);
hipError_t launch_sketch2(const vkv_sketch2_args &a, const Sketch2Layout &L,
                          hipStream_t s);

// ------------------------------------------------------------ maintenance
hipError_t launch_append(const vkv_append_args &a, uint16_t *host_kv_dev,
                         hipStream_t s);

// ------------------------------------------------------------ dense baselines
struct DenseLayout {
  int parts;
  size_t pm, pd, po, total;
};

DenseLayout dense_layout(const vkv_dense_args &a);
hipError_t launch_dense(const vkv_dense_args &a, const DenseLayout &L,
                        const uint16_t *kv_dev, hipStream_t s);

}  // namespace vkv
