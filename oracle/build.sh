#!/bin/sh
# Builds the fp64 CPU oracle (test infrastructure) next to this script.
set -e
cd "$(dirname "$0")"
gcc -O2 -fopenmp -fPIC -shared -Wall -Wextra -std=c11 -o liboracle_conv3x3.so conv3x3_oracle.c -lm
