// qd_step.h -- layout of the decode-step workspace, shared by the host plan
// (qd_api.hip) and the persistent kernel (decode_step.hip).
//
// workspace = [StepHeader | StepOp x n_ops | StepStage x n_stages |
//              release lines | arrival counters | stage inputs]
//   release lines     one 128-byte line per workgroup; word 0 holds the tag
//                     of the last stage whose inputs were released to it
//   arrival counters  per stage, kStepGroups group lines then one global
//                     line (128 bytes each); word 0 counts arrivals, never
//                     reset between launches (every launch adds the same
//                     amounts, so counts are taken modulo the group sizes)
//   stage inputs      per stage, its ops' inputs back to back as dense
//                     32-bit words, two BF16 values each (Q4_0 ops: one f32)
#pragma once
#include <stdint.h>

namespace qd {

constexpr uint32_t kStepMagic = 0x51445354u;  // "QDST"
constexpr int kStepLine = 32;                 // 32-bit words per 128-byte line
constexpr int kStepGroups = 8;                // arrival groups: workgroup b -> b % 8

struct StepOp {            // 64 bytes
  const uint8_t *w;        // affine blob, or Q4_0 stream
  const uint16_t *x;       // BF16 [m, cols] input (Q4_0: f32)
  uint16_t *y;             // BF16 [m, rows] output (Q4_0: f32)
  const void *unused;
  int32_t rows, cols;
  int32_t stage;
  int32_t row_base;        // first row of this op in its stage's row space
  int32_t pad[4];
};

// A stage's input (its ops' inputs back to back, `words` 32-bit words of two
// BF16 each, or of one f32 for Q4_0 ops) is split into slices of 2^lg words;
// workgroup j publishes slice j, words [j*2^lg, (j+1)*2^lg), one word per
// lane.
struct StepStage {         // 32 bytes
  uint32_t *data;          // the stage's input words (dense)
  int32_t op0, nops;       // ops [op0, op0 + nops)
  int32_t rows_total;      // sum of the ops' rows
  int32_t cols;            // shared input width
  int32_t chunks;          // ceil(cols / 1024) (Q4_0: ceil(cols / 2048))
  uint16_t words;          // nops * m * cols / 2 (Q4_0: nops * m * cols; <= 16384)
  uint16_t lg;             // log2 of the slice length (1..6)
};

struct StepHeader {        // 512 bytes
  uint32_t magic;
  int32_t n_ops, n_stages, m, nwg, xmax;
  uint32_t ops_off, stages_off, lds_bytes;
  uint32_t rel_off, ctr_off, data_off;
  uint32_t pad0[52];
  uint32_t epoch;          // byte 256: tag base, advanced by n_stages per launch
  uint32_t pad1[31];
  uint32_t error;          // byte 384: 0 = ok; bit flags from the kernel
  uint32_t pad2[31];
};

static_assert(sizeof(StepOp) == 64, "StepOp layout");
static_assert(sizeof(StepStage) == 32, "StepStage layout");
static_assert(sizeof(StepHeader) == 512, "StepHeader layout");

}  // namespace qd
