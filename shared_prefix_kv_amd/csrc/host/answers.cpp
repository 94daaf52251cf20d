// Answer layer (jdon.com openjev-sglang article, "three question types" and
// "confidence" sections): a yes/no question reports the probability of its
// first ("yes") label, a choice question the most likely option, a score
// question the expectation of the option number counted from 0; the
// confidence of any answer is one minus the distribution's Shannon entropy
// (natural log) divided by ln K, its largest possible value.
#include "answers.hpp"

#include <cmath>

#include "../../../include/jev.h"

namespace jev {

Answer answer(int32_t kind, const float* p, int32_t K) {
  Answer a{0.0, 0, 0.0};
  double expect = 0.0, h = 0.0;
  for (int32_t j = 0; j < K; ++j) {
    const double pj = p[j];
    if (pj > double(p[a.choice])) a.choice = j;  // strict: ties keep the lower index
    expect += double(j) * pj;
    if (pj > 0.0) h -= pj * std::log(pj);  // 0 ln 0 = 0
  }
  a.confidence = 1.0 - h / std::log(double(K));
  if (kind == JEV_ANSWER_NOUL)
    a.value = double(p[0]);
  else if (kind == JEV_ANSWER_CHOICE)
    a.value = double(a.choice);
  else
    a.value = expect;
  return a;
}

}  // namespace jev
