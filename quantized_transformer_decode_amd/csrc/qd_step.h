// qd_step.h -- layout of the decode-step workspace, shared by the host plan
// (qd_api.hip) and the persistent kernel (decode_step.hip).
//
// workspace = [StepHeader | StepOp x n_ops | StepStage x n_stages | staging]
// staging holds, per op, m*cols tagged input words (tag << 16 | BF16 bits).
#pragma once
#include <stdint.h>

namespace qd {

constexpr uint32_t kStepMagic = 0x51445354u;  // "QDST"

struct StepOp {            // 64 bytes
  const uint8_t *w;        // affine blob
  const uint16_t *x;       // BF16 [m, cols] input
  uint16_t *y;             // BF16 [m, rows] output
  uint32_t *stg;           // tagged staging words [m * cols]
  int32_t rows, cols;
  int32_t stage;
  int32_t row_base;        // first row of this op in its stage's row space
  int32_t pad[4];
};

// A stage's input (its ops' inputs back to back, `words` words) is split
// into slices of 2^lg words; slice j is published by workgroup j as words
// [j*2^lg, (j+1)*2^lg) of each staging replica, so the words lie densely and
// a consumer reads whole lines.  Publishers that share a line write disjoint
// 32-bit words (stores carry byte masks; nothing is read back and merged).
struct StepStage {         // 32 bytes
  uint32_t *stg;           // staging: replicas of ceil(words / 2^lg) * 64 words
  int32_t op0, nops;       // ops [op0, op0 + nops)
  int32_t rows_total;      // sum of the ops' rows
  int32_t cols;            // shared input width
  int32_t chunks;          // ceil(cols / 1024)
  uint16_t words;          // nops * m * cols (<= 16384)
  uint16_t lg;             // log2 of the slice length (1..6)
};

struct StepHeader {        // 512 bytes
  uint32_t magic;
  int32_t n_ops, n_stages, m, nwg, xmax;
  uint32_t ops_off, stages_off, lds_bytes;
  uint32_t pad0[55];
  uint32_t epoch;          // byte 256: tag base, advanced by n_stages per launch
  uint32_t pad1[31];
  uint32_t error;          // byte 384: 0 = ok; bit flags from the kernel
  uint32_t pad2[31];
};

static_assert(sizeof(StepOp) == 64, "StepOp layout");
static_assert(sizeof(StepStage) == 32, "StepStage layout");
static_assert(sizeof(StepHeader) == 512, "StepHeader layout");

}  // namespace qd
