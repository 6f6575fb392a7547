// Test driver: reads "theta pos i" lines on stdin and prints the float32
// cos and sin that the decode kernels use for pos * theta^(-2i/128)
// (decode_attention_head_amd/csrc/dah_rope.h), built as plain host C++.
#include <stdio.h>

#include "dah_rope.h"

int main() {
  double theta;
  int pos, i;
  while (scanf("%lf %d %d", &theta, &pos, &i) == 3) {
    const dah::RopePowers rp = dah::rope_powers(theta);
    float c, s;
    dah::rope_cos_sin((double)pos * dah::rope_inv_freq(i, rp), &c, &s);
    printf("%.9e %.9e\n", (double)c, (double)s);
  }
  return 0;
}
