// Answer layer on the host: the post-processing of one branch's label
// distribution by question type, and its confidence.
#pragma once

#include <stdint.h>

namespace jev {

struct Answer {
  double value;      // P(yes), the chosen index, or the expected score
  int32_t choice;    // index of the largest probability (lowest on ties)
  double confidence; // 1 - H(P) / ln K
};

// p: K >= 2 finite, non-negative probabilities in label order; kind: one of
// JEV_ANSWER_NOUL / _CHOICE / _SCORE (validated by the caller).
Answer answer(int32_t kind, const float* p, int32_t K);

}  // namespace jev
